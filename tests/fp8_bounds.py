"""The FP8 forward tests' error bounds (test helper; the derivation is in test_fp8_parity_gpu.py).

Per output row i of one head, with the decoded, descaled values q, k, v, the visible keys J(i), the
weights p_j = softmax_j(scale q_i . k_j), L = sum_j exp(s_j - max s), W_c = sum_j p_j |v_jc| and
dS_i = EPS_MFMA_QK * scale * max_j sum_c |q_ic k_jc|:

    bound_c = 2^-4 W_c + 2^-18 sum_j |v_jc| / L + 2^-8 |O_c| + (1e-3 + EPS_MFMA_PV + 2 dS_i) W_c + 1e-6
    lse bound = dS_i + 1e-5 + 1e-6 |LSE|
    predicted squared error_c = 2^-8 / 6 sum_j p_j^2 v_jc^2 + 2^-16 / 6 O_c^2

``error_model_rows`` evaluates them row by row for selected rows; ``error_model_heads`` evaluates the
same formulas for every row of every head with whole-head matrix products (a CPU test checks that
the two agree).
"""
import numpy as np

import oracle
from fp8_mfma import EPS_MFMA_PV, EPS_MFMA_QK


def _decoded(q8, k8, v8, scales, b, h):
    qd, kd, vd = (float(np.float32(s)) for s in scales)
    return (oracle.e4m3_to_f64(q8[b, h]) * qd, oracle.e4m3_to_f64(k8[b, h]) * kd,
            oracle.e4m3_to_f64(v8[b, h]) * vd)


def error_model_rows(q8, k8, v8, scales, causal, scale, heads_rows):
    """Per selected row: the element bound on O, the bound on LSE and the predicted squared error of O
    (numpy float64). heads_rows: list of (b, h, i)."""
    bounds, lbounds, pred = [], [], []
    cache = {}
    for b, h, i in heads_rows:
        if (b, h) not in cache:
            cache[(b, h)] = _decoded(q8, k8, v8, scales, b, h)
        qf, kf, vf = cache[(b, h)]
        keys = i + 1 if causal else kf.shape[0]
        s = scale * (kf[:keys] @ qf[i])
        ds = EPS_MFMA_QK * scale * float((np.abs(kf[:keys]) @ np.abs(qf[i])).max())
        e = np.exp(s - s.max())
        L = e.sum()
        p = e / L
        av = np.abs(vf[:keys])
        W = p @ av
        o = p @ vf[:keys]
        lse = s.max() + np.log(L)
        bounds.append(2.0 ** -4 * W + 2.0 ** -18 * av.sum(axis=0) / L + 2.0 ** -8 * np.abs(o)
                      + (1e-3 + EPS_MFMA_PV + 2 * ds) * W + 1e-6)
        lbounds.append(ds + 1e-5 + 1e-6 * abs(lse))
        pred.append(2.0 ** -8 / 6 * ((p ** 2) @ (vf[:keys] ** 2)) + 2.0 ** -16 / 6 * o ** 2)
    return np.array(bounds), np.array(lbounds), np.array(pred)


def error_model_heads(q8, k8, v8, scales, causal, scale):
    """The same bounds for every row: ``(bound [B,H,T,d], lse bound [B,H,T], predicted squared error
    [B,H,T,d])``, one head at a time (T x T float64 matrices per head)."""
    B, H, T, d = q8.shape
    bound, lbound, pred = np.empty((B, H, T, d)), np.empty((B, H, T)), np.empty((B, H, T, d))
    hidden = ~np.tril(np.ones((T, T), dtype=bool)) if causal else np.zeros((T, T), dtype=bool)
    for b in range(B):
        for h in range(H):
            qf, kf, vf = _decoded(q8, k8, v8, scales, b, h)
            s = scale * (qf @ kf.T)
            np.putmask(s, hidden, -np.inf)
            m = s.max(axis=1)
            # exponents below -300 are clamped there (weights under 1e-130 vanish in every sum
            # below; the clamp keeps p^2 out of float64's slow subnormal range)
            s -= m[:, None]
            np.maximum(s, -300.0, out=s)
            p = np.exp(s, out=s)
            np.putmask(p, hidden, 0.0)
            L = p.sum(axis=1)
            p /= L[:, None]
            a = np.abs(qf) @ np.abs(kf).T
            np.putmask(a, hidden, 0.0)
            ds = EPS_MFMA_QK * scale * a.max(axis=1)
            del a
            av = np.abs(vf)
            W = p @ av
            o = p @ vf
            lse = m + np.log(L)
            sum_av = np.cumsum(av, axis=0) if causal else np.broadcast_to(av.sum(axis=0), (T, d))
            bound[b, h] = (2.0 ** -4 * W + 2.0 ** -18 * sum_av / L[:, None] + 2.0 ** -8 * np.abs(o)
                           + (1e-3 + EPS_MFMA_PV + 2 * ds[:, None]) * W + 1e-6)
            lbound[b, h] = ds + 1e-5 + 1e-6 * np.abs(lse)
            p *= p
            pred[b, h] = 2.0 ** -8 / 6 * (p @ (vf ** 2)) + 2.0 ** -16 / 6 * o ** 2
    return bound, lbound, pred

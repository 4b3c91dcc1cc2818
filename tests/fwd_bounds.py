"""The bf16 forward's per-element error bound, derived from its arithmetic (test helper).

The stated tolerance (|dO| <= 1.5e-2, |dLSE| <= 1e-3) is absolute; where |O| is small (small scales,
long near-uniform rows) it admits errors the size of O. This bound follows the kernel's roundings
instead. Per row i of a head, with the visible keys J (n of them, in ceil(n / 64) tiles), the exact
weights p_j = softmax_j(s_ij), s_ij = scale q_i . k_j, O = sum_j p_j v_j and W_c = sum_j p_j |v_jc|:

- scores: the MFMA chain over the head dimension adds d products in fp32, off by at most
  EPS_BF16_QK * sum_c |q_ic k_jc| (times scale); the fp32 scaling by scale * log2(e) and the
  FMA with the running max add 2^-21 (|s_ij| + |m_i|). A weight p_j = exp(s_j - m) carries both
  the error of s_j and that of the max, and exp2 is within 2 ulp: relative error
  eta_i <= 2 (dS_i + dA_i) + 2^-21;
- the weights are rounded to bf16 before P V: at most 2^-8 W_c (bf16 keeps 8 significant bits; the
  row sum l adds the unrounded fp32 weights);
- fp32 sums: l over n weights, its rescales (one per tile) and the P V chain over n keys:
  relative (n + n / 64 + 2) 2^-23 + n EPS_BF16_SUM, applied to W_c + |O_c|;
- O is rounded to bf16 once: 2^-8 |O_c|.

    |dO_c| <= 1.01 (2^-8 |O_c| + 2^-8 W_c + (eta_i + sums_i) (W_c + |O_c|)) + 1e-7
    |dLSE_i| <= 1.01 (dS_i + dA_i + (n + n / 64 + 2) 2^-23 + 2^-21 (|m_i| + ln L_i + |LSE_i|)) + 1e-7

(m_i the row max of the scores and L_i = sum_j exp(s_ij - m_i): LSE is formed as m + log l in fp32.)

EPS_BF16_SUM is the textbook bound per addition of a recursive fp32 sum (rounded once per
addition, to nearest or toward zero), used for the long P V chain. EPS_BF16_QK bounds the score
chain (d = 64 or 128 products) per unit of sum |q k|: the textbook d 2^-23 would dominate the bound
at scale 1, and the instruction, measured on the forward's operands, stays within 9.2e-8 (0.39 of
2^-22). tests/test_bf16_mfma_accuracy_gpu.py checks both on the device. A CPU test checks that the
bound holds for a float64 simulation of these roundings and is sharper than the stated tolerance.
"""
import numpy as np

from exact_tiled_attention_07_amd.inputs import bf16_bits_to_f32

EPS_BF16_SUM = 2.0 ** -23  # per addition of a recursive fp32 sum (the P V chain over the keys)
EPS_BF16_QK = 2.0 ** -22   # per unit of sum_c |q_c k_c|, the score chain over the head dimension


def element_bounds(qb, kb, vb, causal, scale, block_mask=None, bm=128, bn=64):
    """(bound on |dO| [B,H,T,d], bound on |dLSE| [B,H,T]) for bf16 inputs (uint16 bits [B,H,T,d]),
    one head at a time with T x T float64 matrices (for the moderate T of the tests using it).
    block_mask (uint8 [1 or B*H, ceil(T/bm), ceil(T/bn)], the block-sparse forward's) hides the
    blocks it does not set; rows that see no key get an infinite bound (they are checked for
    exactness on their own)."""
    B, H, T, d = qb.shape
    bo, bl = np.empty((B, H, T, d)), np.empty((B, H, T))
    causal_hidden = ~np.tril(np.ones((T, T), dtype=bool)) if causal else np.zeros((T, T), dtype=bool)
    for b in range(B):
        for h in range(H):
            hidden = causal_hidden
            if block_mask is not None:
                mh = block_mask[0 if block_mask.shape[0] == 1 else b * H + h].astype(bool)
                hidden = hidden | ~np.repeat(np.repeat(mh, bm, axis=0), bn, axis=1)[:T, :T]
            n = (~hidden).sum(axis=1).astype(np.float64)
            live = n > 0
            n = np.maximum(n, 1.0)
            sums = (n + np.ceil(n / 64) + 2) * 2.0 ** -23
            q, k, v = (bf16_bits_to_f32(x[b, h]).astype(np.float64) for x in (qb, kb, vb))
            s = scale * (q @ k.T)
            abs_s = np.abs(s)
            np.putmask(abs_s, hidden, 0.0)
            np.putmask(s, hidden, -np.inf)
            m = np.where(live, s.max(axis=1), 0.0)
            a = np.abs(q) @ np.abs(k).T
            np.putmask(a, hidden, 0.0)
            ds = EPS_BF16_QK * abs(scale) * a.max(axis=1)
            da = 2.0 ** -21 * (abs_s.max(axis=1) + np.abs(m))
            del a, abs_s
            s -= m[:, None]
            p = np.exp(s, out=s)
            np.putmask(p, hidden, 0.0)
            L = np.where(live, p.sum(axis=1), 1.0)
            p /= L[:, None]
            W = p @ np.abs(v)
            o = p @ v
            lse = m + np.log(L)
            eta = 2 * (ds + da) + 2.0 ** -21
            rel = (eta + sums + n * EPS_BF16_SUM)[:, None]
            bo[b, h] = 1.01 * (2.0 ** -8 * (np.abs(o) + W) + rel * (W + np.abs(o))) + 1e-7
            bl[b, h] = 1.01 * (ds + da + sums + 2.0 ** -21 * (np.abs(m) + np.log(L) + np.abs(lse))) + 1e-7
            bo[b, h][~live] = np.inf
            bl[b, h][~live] = np.inf
    return bo, bl


def check_bounds(o_gpu, lse_gpu, o_ref, lse_ref, bounds):
    """Ratios of the errors to the bound: (worst over O, worst over LSE)."""
    bo, bl = bounds
    fo, fl = np.isfinite(bo), np.isfinite(bl)  # rows that see no key are checked on their own
    ro = np.abs(np.asarray(o_gpu, dtype=np.float64)[fo] - np.asarray(o_ref)[fo]) / bo[fo]
    rl = np.abs(np.asarray(lse_gpu, dtype=np.float64)[fl] - np.asarray(lse_ref)[fl]) / bl[fl]
    return float(ro.max(initial=0.0)), float(rl.max(initial=0.0))

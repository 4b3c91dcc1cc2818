"""Parity of the FP8 forward (fa_fwd_fp8, through the C-ABI) with the CPU oracle on the same FP8
codes (exact attention of the dequantized values in float64).

Tolerance, derived from the arithmetic. The kernel's one added rounding is that of the weights
p'_j = 2^8 exp(s_j - m) to E4M3 before the second product: a relative error of at most 2^-4 for
p'_j >= 2^-6 and an absolute error of at most 2^-10 below (the subnormal spacing is 2^-9). With
l' = sum p'_j = 2^8 L and W_c = sum_j p_j |v_jc| (p normalised), each output element obeys

    |O_gpu - O| <= 2^-4 W_c + 2^-18 sum_j |v_jc| / L + 2^-8 |O| + 1e-3 W_c + 1e-6,

where 2^-8 |O| is the final bf16 rounding (8 significant bits) and 1e-3 W_c covers fp32 accumulation over up to 16384
terms (n u = 16384 x 6e-8) and the fp32 score factor.

The FP8 MFMA does not add its 64 products exactly in fp32: it truncates products far below the
largest nominal exponent of their group. Measured on the device (tests/test_fp8_mfma_accuracy_gpu.py,
which runs with these tests) on the operands this kernel gives it, its result differs from the exact
dot product by at most 5.3e-5 x sum_k |a_k b_k| for the scores (quantized normal rows) and 5.4e-4 x
sum_k |a_k b_k| for P V (E4M3 weights spanning 2^8 down to the subnormals); the tests take
EPS_MFMA_QK = 2^-12 and EPS_MFMA_PV = 2^-10 (tests/fp8_mfma.py), and the accuracy test asserts both.
A score s_j = scale q_i . k_j then carries an error of at most
dS_i = EPS_MFMA_QK * scale * q_descale * k_descale * max_j sum_c |q8_ic k8_jc|, which moves LSE by at
most dS_i (logsumexp is 1-Lipschitz in the max norm) and each weight p_j by a factor within
exp(+-2 dS_i); the product P.V adds EPS_MFMA_PV W_c. So the element bound gains
(2 dS_i + EPS_MFMA_PV) W_c and LSE is checked against dS_i + 1e-5 + 1e-6 |LSE|. The bounds are checked
element by element.
It is loose because rounding errors cancel, so the mean square error is also checked against its
expectation: RNE to 3 mantissa bits has E[rel^2] = 2^-8 / 6 (relative error uniform within half an
ulp, mantissa fraction uniform), so E[(O_gpu - O)_c^2] = 2^-8 / 6 sum_j p_j^2 v_jc^2 (+ the bf16
rounding's 2^-16 / 6 O_c^2, the same formula at 7 mantissa bits); the measured mean over all elements must stay below 3 times the predicted mean. LSE uses the
fp32 weights (not the rounded ones): its error is that of the scores.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import exact_tiled_attention_07_amd as fa
from exact_tiled_attention_07_amd.inputs import WORKLOADS, make_qkv_fp8

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
from fp8_bounds import error_model_heads, error_model_rows  # noqa: E402
MSE_FACTOR = 3.0


def say(msg):
    print(msg, flush=True)


def run_gpu(q8, k8, v8, scales, causal, scale):
    t = [torch.from_numpy(x).to(DEV) for x in (q8, k8, v8)]
    o, lse = fa.fwd_fp8(*t, *scales, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check(q8, k8, v8, scales, causal, scale, label, rows=None):
    """rows=None: every row, against the whole-head oracle (bounds from whole-head products);
    else the listed (b, h, i) rows, against the oracle's row entry."""
    B, H, T, d = q8.shape
    say(f"[gpu fp8] {label} shape={q8.shape} causal={causal} scale={scale}")
    o, lse = run_gpu(q8, k8, v8, scales, causal, scale)
    if rows is None:
        o_ref, lse_ref = oracle.attention_fwd_fp8(q8, k8, v8, causal, scale, *scales)
        o_ref, lse_ref = o_ref.reshape(-1, d), lse_ref.reshape(-1)
        bound, lbound, pred = (x.reshape(-1, d) if x.ndim == 4 else x.reshape(-1)
                               for x in error_model_heads(q8, k8, v8, scales, causal, scale))
        got_o, got_l = o.reshape(-1, d), lse.reshape(-1)
    else:
        bound, lbound, pred = error_model_rows(q8, k8, v8, scales, causal, scale, rows)
        got_o = np.stack([o[b, h, i] for b, h, i in rows])
        got_l = np.array([lse[b, h, i] for b, h, i in rows])
        o_ref, lse_ref = oracle.attention_fwd_fp8_rows(q8, k8, v8, causal, scale, *scales, rows)
    err = np.abs(got_o - o_ref)
    lerr = np.abs(got_l - lse_ref)
    mse, pmse = float((err ** 2).mean()), float(pred.mean())
    say(f"[gpu fp8] {label} max|dO| {err.max():.3e} max ratio to bound {(err / bound).max():.3f} "
        f"mse {mse:.3e} predicted {pmse:.3e} max|dLSE| {lerr.max():.2e} (ratio {(lerr / lbound).max():.3f})")
    assert np.isfinite(got_o).all() and np.isfinite(got_l).all()
    assert np.all(err <= bound), f"{label}: element bound exceeded"
    assert mse <= MSE_FACTOR * pmse, f"{label}: mse {mse} vs predicted {pmse}"
    assert np.all(lerr <= lbound), f"{label}: lse {lerr.max()}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 127, 129, 255, 1000])
def test_fp8_ragged_and_tiny_lengths(T, causal, d):
    q8, k8, v8, scales = make_qkv_fp8(1, 2, T, d, seed=8000 + T + d)
    check(q8, k8, v8, scales, causal, 1.0 / math.sqrt(d), f"T={T} d={d}")


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_fp8_configs(name):
    wl = WORKLOADS[name]
    q8, k8, v8, scales = make_qkv_fp8(wl.B, wl.H, wl.T, wl.d, wl.seed, wl.sigma)
    check(q8, k8, v8, scales, wl.causal, wl.scale, wl.name + " fp8")


def test_fp8_c4_every_row():
    # the FP8 forward as the bench times it on the causal T = 4096 workload (E4M3 copies of its
    # sigma-2 inputs): all 48 heads, every row
    wl = WORKLOADS["c4"]
    q8, k8, v8, scales = make_qkv_fp8(wl.B, wl.H, wl.T, wl.d, wl.seed, wl.sigma)
    check(q8, k8, v8, scales, wl.causal, wl.scale, wl.name + " fp8 (every row)")


@pytest.mark.parametrize("name", ["c4", "c5a", "c5b"])
def test_fp8_full_size_sampled_rows(name):
    wl = WORKLOADS[name]
    q8, k8, v8, scales = make_qkv_fp8(wl.B, wl.H, wl.T, wl.d, wl.seed, wl.sigma)
    rng = np.random.default_rng(17)
    rows = [(int(b), int(h), int(i)) for b, h, i in zip(rng.integers(0, wl.B, 40), rng.integers(0, wl.H, 40),
                                                      rng.integers(0, wl.T, 40))]
    rows += [(0, 0, 0), (0, 0, 63), (0, 0, 64), (wl.B - 1, wl.H - 1, wl.T - 1), (1, 2, 4095)]
    rows = sorted(set(rows))
    check(q8, k8, v8, scales, wl.causal, wl.scale, wl.name + " fp8 sampled", rows=rows)


def test_fp8_long_head_sampled_rows():
    # one head of 2^18 queries and keys (the last Q block walks 4096 K/V tiles), causal, sampled rows
    T = 1 << 18
    q8, k8, v8, scales = make_qkv_fp8(1, 1, T, 64, seed=18, sigma=2.0)
    rng = np.random.default_rng(18)
    rows = sorted({(0, 0, int(i)) for i in [0, 1, 63, 64, 127, 128, T // 2, T - 2, T - 1]
                   + rng.integers(0, T, 20).tolist()})
    check(q8, k8, v8, scales, True, 0.125, "T=2^18 fp8 sampled", rows=rows)


def test_fp8_causal_head_groups():
    # B4 H16 T32768 d64, causal: with one-byte K and V a head holds 4 MB of K/V, so each XCD takes its
    # 8 heads 4 at a time (the K/V budget of causal launches). Every row is written (the outputs start
    # as NaN) and rows sampled in the heads on both sides of the group boundary (heads 0..31 form
    # every XCD's first group, 32..63 its second) satisfy the error bounds against the oracle
    B, H, T, d = 4, 16, 32768, 64
    q8, k8, v8, scales = make_qkv_fp8(B, H, T, d, seed=19)
    say(f"[gpu fp8] causal head groups B{B} H{H} T{T} d{d}")
    t = [torch.from_numpy(x).to(DEV) for x in (q8, k8, v8)]
    o = torch.full((B, H, T, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, H, T), float("nan"), dtype=torch.float32, device=DEV)
    fa.fwd_fp8(*t, *scales, causal=True, scale=0.125, out=o, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any().item() and not torch.isnan(lse).any().item()
    rng = np.random.default_rng(19)
    rows = sorted({(bh // H, bh % H, int(i)) for bh in (0, 31, 32, 63)
                   for i in [0, 1, 63, 64, T // 2, T - 1] + rng.integers(0, T, 6).tolist()})
    got_o = np.stack([o[b, h, i].float().cpu().numpy().astype(np.float64) for b, h, i in rows])
    got_l = np.array([float(lse[b, h, i]) for b, h, i in rows])
    bound, lbound, pred = error_model_rows(q8, k8, v8, scales, True, 0.125, rows)
    o_ref, lse_ref = oracle.attention_fwd_fp8_rows(q8, k8, v8, True, 0.125, *scales, rows)
    err, lerr = np.abs(got_o - o_ref), np.abs(got_l - lse_ref)
    say(f"[gpu fp8] head groups max ratio to bound {(err / bound).max():.3f} lse ratio {(lerr / lbound).max():.3f}")
    assert np.all(err <= bound) and np.all(lerr <= lbound)
    assert float((err ** 2).mean()) <= MSE_FACTOR * float(pred.mean())


def test_fp8_scales_and_descales():
    q8, k8, v8, scales = make_qkv_fp8(2, 2, 300, 64, seed=81)
    check(q8, k8, v8, scales, True, 0.01, "scale 0.01")
    check(q8, k8, v8, scales, False, 1.0, "scale 1")
    check(q8, k8, v8, (scales[0] * 4, scales[1] * 3, scales[2] * 0.5), True, 0.125, "descales x4 x3 x0.5")


def test_fp8_closed_forms():
    T = 200
    q8, k8, v8, scales = make_qkv_fp8(1, 2, T, 64, seed=83)
    # causal row 0 sees key 0 only: O[0] = v_descale * e4m3(V[0]) rounded to bf16, exactly
    o, lse = run_gpu(q8, k8, v8, scales, True, 0.125)
    v0 = oracle.e4m3_to_f64(v8[:, :, 0]) * float(np.float32(scales[2]))
    ref = torch.from_numpy(v0.astype(np.float32)).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(o[:, :, 0], ref)
    # Q = 0: every weight equal; causal row i is the mean of V[0..i]
    qz = np.zeros_like(q8)
    o, lse = run_gpu(qz, k8, v8, scales, True, 0.125)
    vf = oracle.e4m3_to_f64(v8) * float(np.float32(scales[2]))
    mean = np.cumsum(vf, axis=2) / np.arange(1, T + 1)[None, None, :, None]
    np.testing.assert_allclose(o, mean, rtol=2.0 ** -8, atol=1e-6)
    np.testing.assert_allclose(lse, np.log(np.arange(1, T + 1))[None, None, :] * np.ones((1, 2, 1)), atol=1e-5)


def test_fp8_writes_stay_inside_outputs_and_are_deterministic():
    B, H, T, d = 2, 3, 333, 64
    q8, k8, v8, scales = make_qkv_fp8(B, H, T, d, seed=85)
    t = [torch.from_numpy(x).to(DEV) for x in (q8, k8, v8)]
    n, nl, guard = B * H * T * d, B * H * T, 4096
    big = torch.full((n + 2 * guard,), float("nan"), dtype=torch.bfloat16, device=DEV)
    lbig = torch.full((nl + 2 * guard,), float("nan"), dtype=torch.float32, device=DEV)
    o, lse = big[guard:guard + n].view(B, H, T, d), lbig[guard:guard + nl].view(B, H, T)
    fa.fwd_fp8(*t, *scales, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isnan(big[:guard].float()).all() and torch.isnan(big[guard + n:].float()).all()
    assert torch.isnan(lbig[:guard]).all() and torch.isnan(lbig[guard + nl:]).all()
    o2, l2 = fa.fwd_fp8(*[x.view(torch.float8_e4m3fn) for x in t], *scales)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, l2)


def test_fp8_binding_rejects():
    q = torch.zeros(1, 1, 8, 64, dtype=torch.uint8, device=DEV)
    with pytest.raises(TypeError):
        fa.fwd_fp8(q.to(torch.int8), q, q, 1.0, 1.0, 1.0)
    with pytest.raises(fa.FaError):
        fa.fwd_fp8(q, q, q, 0.0, 1.0, 1.0)
    with pytest.raises(ValueError):
        fa.fwd_fp8(q, q[:, :, :4].contiguous(), q, 1.0, 1.0, 1.0)
    with pytest.raises(ValueError):  # outputs on another device than the inputs
        fa.fwd_fp8(q, q, q, 1.0, 1.0, 1.0, out=torch.empty(1, 1, 8, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        fa.fwd_fp8(q, q, q, 1.0, 1.0, 1.0, lse=torch.empty(1, 1, 8, dtype=torch.float32))

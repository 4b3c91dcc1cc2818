"""Parity of the gfx950 backward (fa_bwd, through the C-ABI) with the CPU fp64 backward oracle.

The GPU backward takes the GPU forward's O and LSE (as a training step would); the oracle recomputes
everything from the bf16 Q, K, V and dO in fp64. Tolerance (derived from the arithmetic, see
``grad_tolerance``): the algorithm must use the forward's bf16 O in D = dO . O, round P and dS to
bf16 before the matrix products, and round the gradients to bf16 at the end. A CPU model of exactly
those roundings (tests/bwd_rounding_model.py, its figures stored in tests/golden/ and recomputed by a
CPU test) reaches an element error of 0.108 (|ref| + rms of the head) in dQ for the sigma-4 scores
(the dominant weight's dS is a small difference of two large terms, and the rounding of O enters
through D) and an RMS error of 0.59% of the RMS. The bounds are twice the model's figures
(tests/bwd_tolerance.py).

Where a gradient is exactly zero by cancellation, the relative bounds say nothing, so there both
checks also admit an absolute floor. That happens on the rows with one visible key (dS = P (dP - D)
with P = 1 and dP = D): dQ's row 0 of a causal head, and every row of a one-token head (dK's too).
dP and D are fp32 sums of d products, each off by at most d 2^-24 sum_c |dO_c| max|v|, and the rows
of P sum to one, so dQ = scale dS K (dK = scale dS^T Q) is off by at most 2 scale d 2^-24 max|k|
(max|q|) times that. Every other element is held to the relative bounds alone. Every element
also has the floor 64 * 2^-126: an exact gradient below 2^-126, the smallest normal fp32 (and bf16)
number (a weight of exp(-300) times a small difference), cannot be represented by fp32 arithmetic
at all, and near it the kernels' flushed subnormal intermediates lose up to one such unit per term.

Where the relative bounds still fail (a short head whose rows are all dominated by one key, or whose
D values are all small), the error that the forward's rounded O causes through D = dO . O is
computed from the O the backward read and admitted with a 10% margin
(bwd_tolerance.o_rounding_allowance); tests below keep the cases randomised runs found.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import exact_tiled_attention_07_amd as fa
from exact_tiled_attention_07_amd.inputs import WORKLOADS, bf16_bits_from_f32, bf16_bits_to_f32, make_qkv, to_torch_bf16

from bwd_rounding_model import grad_stats
from parity import record_bwd

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
# |gpu - ref| <= ELEM_TOL * (|ref| + rms of the reference over its head), and rms(gpu - ref) <=
# RMS_TOL * rms(ref) per tensor: twice the rounding model's worst figures (tests/bwd_tolerance.py)
from bwd_tolerance import ELEM_TOL, RMS_TOL, o_rounding_allowance  # noqa: E402

FP32_MIN_NORMAL = 2.0 ** -126  # below it an exact gradient is not representable in fp32 or bf16
# the floor every element gets: fp32 subnormal intermediates are flushed to zero, so a sum of up to
# 64 terms near the smallest normal number can be off by 64 of them
UNDERFLOW_FLOOR = 64 * FP32_MIN_NORMAL


def say(msg):
    print(msg, flush=True)


def grad_tolerance(name, gpu, ref, atol=0.0, allowance=None):
    """Element and RMS check of one gradient tensor [B, H, T, d] (or delta [B, H, T]); atol is the
    absolute floor of the fp32 cancellation in dS (see the module docstring). Where the relative
    bounds fail, `allowance()` (dQ, dK and D) gives the per-element bound on what the forward's
    rounded O does through D (bwd_tolerance.o_rounding_allowance), admitted with a 10% margin."""
    atol = atol + UNDERFLOW_FLOOR
    stats = grad_stats(gpu, ref, atol)
    if allowance is not None and (stats["max_ratio"] > ELEM_TOL or stats["rms_ratio"] > RMS_TOL):
        stats = dict(grad_stats(gpu, ref, atol + 1.1 * allowance()), o_rounding_allowance=True)
    assert stats["nonfinite"] == 0, (name, stats)
    assert stats["max_ratio"] <= ELEM_TOL, (name, stats)
    assert stats["rms_ratio"] <= RMS_TOL, (name, stats)
    return stats


def cancellation_floors(qb, kb, vb, dob, causal, scale, i):
    """The absolute floors of dQ, dK, dV and D for rows at positions i (an array broadcastable to the
    rows compared): the fp32 cancellation bound on the rows with one visible key, zero elsewhere."""
    T = qb.shape[2]
    q, k, v, do = (np.abs(bf16_bits_to_f32(x).astype(np.float64)) for x in (qb, kb, vb, dob))
    d = q.shape[-1]
    cancel = d * 2.0 ** -24 * float(do.sum(axis=-1).max(initial=0.0)) * float(v.max(initial=0.0))
    i = np.asarray(i)
    one_key_q = (i == 0) & (causal or T == 1)  # query rows with one visible key
    one_key_k = np.full(i.shape, T == 1)        # key rows seen only by queries that see one key
    return (2 * scale * float(k.max(initial=0.0)) * cancel * one_key_q[..., None],
            2 * scale * float(q.max(initial=0.0)) * cancel * one_key_k[..., None], 0.0, 0.0)


def run_gpu(qb, kb, vb, dob, causal, scale, with_o=False):
    q, k, v, do = (to_torch_bf16(x, DEV) for x in (qb, kb, vb, dob))
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv, delta = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    out = [t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv, delta)]
    return (out, o.float().cpu().numpy().astype(np.float64)) if with_o else out


def allowances(qb, kb, vb, dob, causal, scale, o_used):
    """Lazy per-tensor allowance callables for grad_tolerance (computed at most once)."""
    memo = []

    def get(i):
        if not memo:
            memo.extend(o_rounding_allowance(qb, kb, vb, dob, causal, scale, o_used))
        return memo[i]

    return (lambda: get(0), lambda: get(1), None, lambda: get(2))


def check(qb, kb, vb, dob, causal, scale, label, keep=False):
    say(f"[gpu bwd] {label} shape={qb.shape} causal={causal} scale={scale}")
    got, o_gpu = run_gpu(qb, kb, vb, dob, causal, scale, with_o=True)
    ref = oracle.attention_bwd(qb, kb, vb, dob, causal, scale)
    floors = cancellation_floors(qb, kb, vb, dob, causal, scale, np.arange(qb.shape[2]).reshape(1, 1, -1))
    extra = allowances(qb, kb, vb, dob, causal, scale, o_gpu)
    stats = {n: grad_tolerance(n, g, r, a, x)
             for n, g, r, a, x in zip(("dq", "dk", "dv", "delta"), got, ref, floors, extra)}
    say(f"[gpu bwd] {label} " + " ".join(f"{n}: {s['max_ratio']:.4f}/{s['rms_ratio']:.4f}"
                                         for n, s in stats.items()))
    if keep:
        record_bwd(label, stats)
    return got, ref


def inputs(B, H, T, seed, sigma=1.0, d=64):
    qb, kb, vb = make_qkv(B, H, T, d, seed=seed, sigma=sigma)
    dob, _, _ = make_qkv(B, H, T, d, seed=seed + 7919)
    return qb, kb, vb, dob


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("T", [1, 2, 31, 63, 64, 65, 127, 128, 129, 255, 257, 1000])
def test_bwd_ragged_and_tiny_lengths(T, causal):
    check(*inputs(1, 3, T, 2000 + T), causal, 0.125, f"T={T}")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("T", [1, 2, 63, 65, 128, 129, 257, 1000])
def test_bwd_head_dim_128(T, causal):
    check(*inputs(1, 3, T, 3000 + T, d=128), causal, 1.0 / math.sqrt(128), f"d=128 T={T}")


def test_bwd_head_dim_128_long_and_wide_scores():
    # two heads of the non-causal d = 128 workload's shape at T = 2048, then sigma-2 causal inputs
    check(*inputs(1, 2, 2048, 6, d=128), False, 1.0 / math.sqrt(128), "d=128 T=2048 non-causal")
    check(*inputs(1, 2, 1500, 7, sigma=2.0, d=128), True, 1.0 / math.sqrt(128), "d=128 T=1500 sigma2")


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_bwd_configs(name):
    wl = WORKLOADS[name]
    qb, kb, vb = wl.make()
    dob, _, _ = make_qkv(wl.B, wl.H, wl.T, wl.d, seed=wl.seed + 7919)
    check(qb, kb, vb, dob, wl.causal, wl.scale, wl.name, keep=True)


def test_bwd_c4_every_element():
    # the backward as the bench times it: all 48 heads of the causal T = 4096 workload (its sigma-2
    # inputs), dO drawn from the workload's seed + 7919; every element of dQ, dK, dV and D
    wl = WORKLOADS["c4"]
    qb, kb, vb = wl.make()
    dob, _, _ = make_qkv(wl.B, wl.H, wl.T, wl.d, seed=wl.seed + 7919)
    check(qb, kb, vb, dob, wl.causal, wl.scale, f"{wl.name} (every element)", keep=True)


def test_bwd_d128_workload_first_heads():
    # the d = 128 backward as the bench times it (non-causal B4 H16 T8192, dO from the workload's
    # seed + 7919), the whole call on the GPU; every element of its first 16 heads (a quarter of the
    # call: the oracle's fp64 work for all 64 heads would take minutes)
    wl = WORKLOADS["c5b"]
    qb, kb, vb = wl.make()
    dob, _, _ = make_qkv(wl.B, wl.H, wl.T, wl.d, seed=wl.seed + 7919)
    label = f"{wl.name} heads 0-15 (every element)"
    say(f"[gpu bwd] {label}")
    got = run_gpu(qb, kb, vb, dob, wl.causal, wl.scale)
    sel = [x[:1] for x in (qb, kb, vb, dob)]  # batch 0 = heads 0-15
    ref = oracle.attention_bwd(*sel, wl.causal, wl.scale)
    floors = cancellation_floors(*sel, wl.causal, wl.scale, np.arange(wl.T).reshape(1, 1, -1))
    stats = {n: grad_tolerance(n, g[:1], r, a)
             for n, g, r, a in zip(("dq", "dk", "dv", "delta"), got, ref, floors)}
    say(f"[gpu bwd] {label} " + " ".join(f"{n}: {s['max_ratio']:.4f}/{s['rms_ratio']:.4f}"
                                         for n, s in stats.items()))
    record_bwd(label, stats)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T", [2, 3, 17])
def test_bwd_heads_dominated_by_one_key(T, d, causal):
    # short heads at scale 1: every row's weights are dominated by one key, dQ and dK are near zero
    # and their error is the forward's rounded O seen through D; the relative bounds alone fail
    # here, and the allowance for that rounding (bwd_tolerance.o_rounding_allowance) must cover it.
    # (B1 H1 T2 d64, non-causal, inputs of seeds 0 and 1 is the case a randomised run found.)
    qb, kb, vb = make_qkv(1, 1, T, d, seed=0)
    dob, _, _ = make_qkv(1, 1, T, d, seed=1)
    check(qb, kb, vb, dob, causal, 1.0, f"one-key-dominated T={T} d={d}")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("sigma,scale,vmul", [(8.0, 3.0, 1.0), (4.0, 1.0, 100.0), (1.0, 0.125, 0.01)])
def test_bwd_extreme_magnitudes(sigma, scale, vmul, causal):
    # scores in the thousands, V times 100 or times 0.01: the backward's tolerance is relative to
    # each head's own scale (plus the allowance for heads dominated by one key), so it holds here too
    qb, kb, vb, dob = inputs(1, 2, 257, 95, sigma=sigma)
    vb = bf16_bits_from_f32((bf16_bits_to_f32(vb) * np.float32(vmul)).astype(np.float32))
    check(qb, kb, vb, dob, causal, scale, f"extreme sigma={sigma} scale={scale} V x{vmul}")


def test_bwd_delta_of_a_two_row_head():
    # D = dO . O with the forward's bf16 O: its error is that rounding alone, and in a head of two
    # rows both D values can be small, so the relative RMS bound alone fails; the allowance for the
    # rounding of O covers D too (a randomised run found this case)
    qb, kb, vb = make_qkv(1, 1, 2, 64, seed=118508)
    dob, _, _ = make_qkv(1, 1, 2, 64, seed=118509)
    check(qb, kb, vb, dob, False, 0.125, "two-row head, D")


def test_bwd_gradients_below_the_fp32_range():
    # two causal tokens at scale 1 and sigma 4: query 1 weighs key 1 by about exp(-280), so the
    # exact dQ and dK of that row are ~1.6e-124, below the smallest normal fp32 number; the GPU
    # returns 0 there, within the representability floor (a randomised run found this case)
    qb, kb, vb = make_qkv(1, 1, 2, 64, seed=2, sigma=4.0)
    dob, _, _ = make_qkv(1, 1, 2, 64, seed=3)
    ref = oracle.attention_bwd(qb, kb, vb, dob, True, 1.0)
    assert 0 < np.abs(ref[1]).max() < FP32_MIN_NORMAL  # the case is what it claims to be
    got, _ = check(qb, kb, vb, dob, True, 1.0, "gradients below the fp32 range")
    assert all(np.isfinite(g).all() for g in got)


def test_bwd_gradients_at_the_edge_of_the_fp32_range():
    # three causal tokens at scale 3 and sigma 2: the exact dK of key 1 is ~4.4e-38, a few times the
    # smallest normal fp32 number, and the GPU's, formed from flushed subnormal terms, is off by
    # ~3e-38; the floor of 64 * 2^-126 admits that (a randomised run found this case)
    qb, kb, vb = make_qkv(1, 1, 3, 64, seed=3, sigma=2.0)
    dob, _, _ = make_qkv(1, 1, 3, 64, seed=4)
    ref = oracle.attention_bwd(qb, kb, vb, dob, True, 3.0)
    assert FP32_MIN_NORMAL < np.abs(ref[1]).max() < UNDERFLOW_FLOOR  # the case is what it claims
    got, _ = check(qb, kb, vb, dob, True, 3.0, "gradients at the edge of the fp32 range")
    assert all(np.isfinite(g).all() for g in got)


def test_bwd_long_sequence():
    # one twelfth of the T = 4096 workload (4 of its 48 heads), inputs at its sigma of 2
    check(*inputs(1, 4, 4096, 4, sigma=2.0), True, 0.125, "T=4096 sigma2 (4 heads)")


@pytest.mark.parametrize("B,H,T,d,causal", [(1, 2, 16384, 64, True), (1, 1, 8192, 128, False)])
def test_bwd_long_heads_sampled_rows(B, H, T, d, causal):
    # long heads (the dK/dV kernel's first key block walks 256 Q tiles at T = 16384) against the
    # row entry of the oracle on sampled query and key rows: first and last rows, tile edges, the
    # middle and random rows of every head
    qb, kb, vb, dob = inputs(B, H, T, 90 + d, sigma=1.5, d=d)
    scale = 1.0 / math.sqrt(d)
    say(f"[gpu bwd] long heads B={B} H={H} T={T} d={d} causal={causal}")
    q, k, v, do = (to_torch_bf16(x, DEV) for x in (qb, kb, vb, dob))
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv, delta = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(T + d)
    rows = sorted({bh * T + i for bh in range(B * H)
                   for i in [0, 1, 63, 64, 127, 128, T // 2, T - 2, T - 1] + rng.integers(0, T, 12).tolist()})
    idx = torch.as_tensor(rows, dtype=torch.int64, device=DEV)
    got = [t.reshape(-1, d).index_select(0, idx).float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv)]
    got.append(delta.reshape(-1).index_select(0, idx).cpu().numpy().astype(np.float64))
    ref = oracle.attention_bwd_rows(qb, kb, vb, dob, causal, scale, rows, rows)
    floors = cancellation_floors(qb, kb, vb, dob, causal, scale, (np.array(rows) % T).reshape(1, 1, -1))
    n = len(rows)
    for name, g, r, a in zip(("dq", "dk", "dv", "delta"), got, ref, floors):
        shape = (1, 1, n, d) if name != "delta" else (1, 1, n)
        st = grad_tolerance(name, g.reshape(shape), r.reshape(shape), a)
        say(f"[gpu bwd] long heads {name}: {st['max_ratio']:.4f}/{st['rms_ratio']:.4f}")


@pytest.mark.parametrize("B,H,T,d", [(4, 16, 8192, 128), (4, 16, 16384, 64)])
def test_bwd_causal_head_groups(B, H, T, d):
    # causal launches whose XCDs take their 8 heads 4 at a time (the K/V budget of causal launches,
    # used by both backward kernels): every gradient row is written (outputs start as NaN) and rows
    # sampled in the heads on both sides of each group boundary (heads 0..31 form every XCD's first
    # group, 32..63 its second) match the row oracle
    assert fa.plan(B, H, T, d, True)["head_group"] == 4
    qb, kb, vb, dob = inputs(B, H, T, 120 + d, d=d)
    scale = 1.0 / math.sqrt(d)
    say(f"[gpu bwd] causal head groups B={B} H={H} T={T} d={d}")
    q, k, v, do = (to_torch_bf16(x, DEV) for x in (qb, kb, vb, dob))
    o, lse = fa.fwd(q, k, v, causal=True, scale=scale)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    delta = torch.full_like(lse, float("nan"))
    fa.bwd(q, k, v, o, lse, do, causal=True, scale=scale, dq=dq, dk=dk, dv=dv, delta=delta)
    torch.cuda.synchronize()
    for t in (dq, dk, dv, delta):
        assert not torch.isnan(t).any().item()
    rng = np.random.default_rng(T + d + 1)
    rows = sorted({bh * T + i for bh in (0, 31, 32, 63)
                   for i in [0, 1, 127, 128, T // 2, T - 1] + rng.integers(0, T, 10).tolist()})
    idx = torch.as_tensor(rows, dtype=torch.int64, device=DEV)
    got = [t.reshape(-1, d).index_select(0, idx).float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv)]
    got.append(delta.reshape(-1).index_select(0, idx).cpu().numpy().astype(np.float64))
    ref = oracle.attention_bwd_rows(qb, kb, vb, dob, True, scale, rows, rows)
    floors = cancellation_floors(qb, kb, vb, dob, True, scale, (np.array(rows) % T).reshape(1, 1, -1))
    n = len(rows)
    for name, g, r, a in zip(("dq", "dk", "dv", "delta"), got, ref, floors):
        shape = (1, 1, n, d) if name != "delta" else (1, 1, n)
        st = grad_tolerance(name, g.reshape(shape), r.reshape(shape), a)
        say(f"[gpu bwd] head groups {name}: {st['max_ratio']:.4f}/{st['rms_ratio']:.4f}")


@pytest.mark.parametrize("causal", [True, False])
def test_bwd_other_scales_and_wide_scores(causal):
    check(*inputs(2, 2, 300, 77), causal, 0.01, "scale=0.01")
    check(*inputs(2, 2, 300, 78), causal, 1.0, "scale=1.0")
    qb, kb, _, dob = inputs(1, 4, 700, 5, sigma=4.0)
    _, _, vb, _ = inputs(1, 4, 700, 6)
    check(qb, kb, vb, dob, causal, 0.125, "sigma4 q/k")


def test_bwd_closed_forms():
    T = 200
    _, kb, vb, dob = inputs(1, 2, T, 21)
    # Q = 0: every dK is an exact zero (dK = scale dS^T Q)
    qz = np.zeros_like(kb)
    got, ref = check(qz, kb, vb, dob, True, 0.125, "Q=0")
    np.testing.assert_array_equal(got[1], 0.0)
    # sum over keys of dV equals the sum over queries of dO (rows of P sum to one)
    qb, kb, vb, dob = inputs(1, 2, T, 22)
    got, _ = check(qb, kb, vb, dob, False, 0.125, "sum dV")
    do = bf16_bits_to_f32(dob).astype(np.float64)
    np.testing.assert_allclose(got[2].sum(axis=2), do.sum(axis=2), rtol=0.02, atol=0.05)
    # all V rows equal: O does not depend on the scores, so dQ and dK vanish up to rounding
    row = np.random.default_rng(3).standard_normal(64).astype(np.float32)
    vconst = bf16_bits_from_f32(np.broadcast_to(row, (1, 2, T, 64)).copy())
    got = run_gpu(qb, kb, vconst, dob, True, 0.125)
    assert np.abs(got[0]).max() < 0.02 and np.abs(got[1]).max() < 0.02, (np.abs(got[0]).max(), np.abs(got[1]).max())


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_writes_stay_inside_outputs_and_are_deterministic(d):
    B, H, T = 2, 3, 333
    qb, kb, vb, dob = inputs(B, H, T, 41, d=d)
    q, k, v, do = (to_torch_bf16(x, DEV) for x in (qb, kb, vb, dob))
    o, lse = fa.fwd(q, k, v, causal=True)
    n, nl, guard = B * H * T * d, B * H * T, 4096
    bigs = [torch.full((n + 2 * guard,), float("nan"), dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    dbig = torch.full((nl + 2 * guard,), float("nan"), dtype=torch.float32, device=DEV)
    dq, dk, dv = (b[guard:guard + n].view(B, H, T, d) for b in bigs)
    delta = dbig[guard:guard + nl].view(B, H, T)
    fa.bwd(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv, delta=delta)
    torch.cuda.synchronize()
    for b in bigs:
        assert torch.isnan(b[:guard].float()).all() and torch.isnan(b[guard + n:].float()).all()
    assert torch.isnan(dbig[:guard]).all() and torch.isnan(dbig[guard + nl:]).all()
    for t in (dq, dk, dv, delta):
        assert torch.isfinite(t.float()).all()
    again = fa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv), again[:3]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(delta, again[3])


def test_bwd_binding_rejects():
    q = torch.zeros(1, 1, 8, 96, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(1, 1, 8, dtype=torch.float32, device=DEV)
    with pytest.raises(fa.FaError):  # the backward takes d = 64 or 128
        fa.bwd(q, q, q, q, lse, q)
    q64 = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        fa.bwd(q64, q64, q64, q64, lse[..., :4], q64)
    with pytest.raises(TypeError):
        fa.bwd(q64, q64, q64, q64.float(), lse, q64)
    with pytest.raises(ValueError):  # lse on another device than q
        fa.bwd(q64, q64, q64, q64, lse.cpu(), q64)

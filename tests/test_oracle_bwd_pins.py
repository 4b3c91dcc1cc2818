"""Pins of the CPU backward oracle against facts that do not come from the oracle itself.

B1 finite differences of the forward: the gradients must be the derivative of the forward map
   L(Q, K, V) = sum(dO * O(Q, K, V)), checked by central differences of the float64 forward.
B2 a library: PyTorch autograd (float64, CPU) through a plain softmax attention.
B3 exact identities of the softmax Jacobian: sum_j dV_j = sum_i dO_i (rows of P sum to one) and
   sum_j dK_j = 0 (each row of dS sums to zero); delta = rowsum(dO * O) with O from the pinned
   forward oracle.
B4 special cases: a single visible key, constant V rows, Q = 0, dO = 0.
B5 the float64 forward used by B1 equals the bf16 forward oracle bit for bit on bf16 inputs, and
   the bf16 backward entry point equals the float64 one on the widened inputs.
B6 the row entry for long heads (numpy) equals the whole-head backward (C, pinned by B1-B5) on
   every query and key row.
A plausible slip in the backward (a dropped delta term, a missing scale, a transposed operand, a
wrong mask bound) fails B1 and B2; B3 catches a dropped normalisation.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_07_amd.inputs import bf16_bits_to_f32, make_qkv


def _rand(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


@pytest.mark.parametrize("causal", [True, False])
def test_b1_finite_differences(causal):
    B, H, T, d, scale = 1, 2, 5, 3, 0.7
    q, k, v, do = (_rand((B, H, T, d), s) for s in (1, 2, 3, 4))
    dq, dk, dv, _ = oracle.attention_bwd_f64(q, k, v, do, causal, scale)

    def loss(qq, kk, vv):
        o, _ = oracle.attention_fwd_f64(qq, kk, vv, causal, scale)
        return float((o * do).sum())

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8, err_msg=f"d{name}")


@pytest.mark.parametrize("causal,d", [(True, 16), (False, 16), (True, 128)])
def test_b2_torch_autograd(causal, d):
    B, H, T, scale = 2, 3, 37, 0.25
    q, k, v, do = (_rand((B, H, T, d), s, 1.5) for s in (11, 12, 13, 14))
    dq, dk, dv, delta = oracle.attention_bwd_f64(q, k, v, do, causal, scale)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = torch.matmul(tq, tk.transpose(-1, -2)) * scale
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), tv)
    o.backward(torch.tensor(do, dtype=torch.float64))
    for name, mine, ref in (("q", dq, tq.grad), ("k", dk, tk.grad), ("v", dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=1e-10, atol=1e-12, err_msg=f"d{name}")
    np.testing.assert_allclose(delta, (o.detach().numpy() * do).sum(-1), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_b3_softmax_jacobian_identities(causal):
    B, H, T, d = 1, 4, 200, 64
    qb, kb, vb = make_qkv(B, H, T, d, seed=21)
    dob, _, _ = make_qkv(B, H, T, d, seed=22)
    dq, dk, dv, delta = oracle.attention_bwd(qb, kb, vb, dob, causal, 0.125)
    do = bf16_bits_to_f32(dob).astype(np.float64)
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), rtol=1e-10, atol=1e-10)
    assert np.abs(dk.sum(axis=2)).max() < 1e-10 * max(1.0, np.abs(dk).max() * T)
    o, _ = oracle.attention_fwd(qb, kb, vb, causal, 0.125)
    np.testing.assert_allclose(delta, (o * do).sum(-1), rtol=1e-12, atol=1e-12)


def test_b4_special_cases():
    rng = np.random.default_rng(5)
    # one visible key (T = 1): P = 1, so dV = dO, and dS = 0 gives dQ = dK = 0
    q, k, v, do = (rng.standard_normal((1, 2, 1, 8)) for _ in range(4))
    dq, dk, dv, delta = oracle.attention_bwd_f64(q, k, v, do, True, 0.3)
    np.testing.assert_array_equal(dq, 0.0)
    np.testing.assert_array_equal(dk, 0.0)
    np.testing.assert_allclose(dv, do, rtol=0, atol=0)
    np.testing.assert_allclose(delta, (do * v).sum(-1), rtol=1e-15)
    # every V row equal: O does not depend on the scores, so dQ = dK = 0 and dV = P^T dO
    T, d = 9, 4
    q, k, do = (rng.standard_normal((1, 1, T, d)) for _ in range(3))
    v = np.broadcast_to(rng.standard_normal(d), (1, 1, T, d)).copy()
    for causal in (True, False):
        dq, dk, dv, _ = oracle.attention_bwd_f64(q, k, v, do, causal, 0.5)
        assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
    # Q = 0: every visible key has the same weight; dK = 0 (it is a sum of dS * q) and, non-causal,
    # dV_j = mean over rows of dO
    q0 = np.zeros((1, 1, T, d))
    v = rng.standard_normal((1, 1, T, d))
    dq, dk, dv, _ = oracle.attention_bwd_f64(q0, k, v, do, False, 0.5)
    np.testing.assert_array_equal(dk, 0.0)
    np.testing.assert_allclose(dv, np.broadcast_to(do.mean(axis=2, keepdims=True), dv.shape), rtol=1e-13)
    dq, dk, dv, _ = oracle.attention_bwd_f64(q0, k, v, do, True, 0.5)
    expect_dv = np.zeros_like(dv)
    for j in range(T):  # causal: key j gets weight 1/(i+1) from every row i >= j
        expect_dv[0, 0, j] = sum(do[0, 0, i] / (i + 1) for i in range(j, T))
    np.testing.assert_allclose(dv, expect_dv, rtol=1e-13)
    # dO = 0: all gradients vanish
    z = np.zeros((1, 1, T, d))
    out = oracle.attention_bwd_f64(q, k, v, z, True, 0.5)
    for g in out:
        np.testing.assert_array_equal(g, 0.0)


def test_b5_f64_paths_match_the_bf16_oracle():
    qb, kb, vb = make_qkv(2, 2, 65, 64, seed=31)
    dob, _, _ = make_qkv(2, 2, 65, 64, seed=32)
    f = [bf16_bits_to_f32(x).astype(np.float64) for x in (qb, kb, vb, dob)]
    for causal in (True, False):
        o16, l16 = oracle.attention_fwd(qb, kb, vb, causal, 0.125)
        o64, l64 = oracle.attention_fwd_f64(f[0], f[1], f[2], causal, 0.125)
        np.testing.assert_array_equal(o16, o64)
        np.testing.assert_array_equal(l16, l64)
        g16 = oracle.attention_bwd(qb, kb, vb, dob, causal, 0.125)
        g64 = oracle.attention_bwd_f64(*f, causal, 0.125)
        for a, b in zip(g16, g64):
            np.testing.assert_array_equal(a, b)


def test_bwd_entry_points_reject_bad_input():
    qb, kb, vb = make_qkv(1, 1, 4, 8, seed=1)
    with pytest.raises(ValueError):
        oracle.attention_bwd(qb, kb, vb[:, :, :3], qb, True, 0.5)
    with pytest.raises(TypeError):
        oracle.attention_bwd(qb.astype(np.float32), kb, vb, qb, True, 0.5)
    with pytest.raises(RuntimeError):
        oracle.attention_bwd(qb, kb, vb, qb, True, math.inf)
    empty = np.zeros((1, 1, 0, 8), dtype=np.uint16)
    out = oracle.attention_bwd(empty, empty, empty, empty, True, 0.5)
    assert all(x.size == 0 for x in out)


@pytest.mark.parametrize("B,H,T,d,causal", [(1, 2, 300, 64, True), (1, 2, 300, 64, False), (2, 1, 130, 128, True),
                                            (1, 1, 1, 64, True), (1, 1, 65, 16, False)])
def test_b6_row_entry_matches_the_whole_head_oracle(B, H, T, d, causal):
    # attention_bwd_rows (numpy, rows) against attention_bwd (C, whole heads, pinned by B1-B5) on
    # every query and key row; the row blocking is made smaller than T to cross block edges
    qb, kb, vb = make_qkv(B, H, T, d, seed=60 + T + d, sigma=1.5)
    dob = make_qkv(B, H, T, d, seed=61 + T)[0]
    scale = d ** -0.5
    dq, dk, dv, delta = oracle.attention_bwd(qb, kb, vb, dob, causal, scale)
    rows = np.arange(B * H * T)
    rq, rk, rv, rd = oracle.attention_bwd_rows(qb, kb, vb, dob, causal, scale, rows, rows[::-1], block_rows=64)
    np.testing.assert_allclose(rq, dq.reshape(-1, d), rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(rk, dk.reshape(-1, d)[::-1], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(rv, dv.reshape(-1, d)[::-1], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(rd, delta.reshape(-1), rtol=1e-10, atol=1e-12)

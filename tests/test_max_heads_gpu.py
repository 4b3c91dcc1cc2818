"""Every entry point that launches one workgroup per (query block, head) at the largest accepted
B*H (FA_MAX_BH = 2^24) with T = 1, through the C-ABI.

At 2^24 workgroups of 256 threads the grid holds 2^32 work-items, one more than a dispatch dimension
counts, so the library folds the grid into two dimensions; these tests check that every head is
computed exactly once. With a single key the softmax weight is exp(0) = 1 (the closed form for T = 1:
O equals V, LSE is the one scaled score; learn-llm.fim.ai "手写 FlashAttention：拆开 SDPA 这个黑盒",
STEP 1), so outputs are checked bit for bit against V where that is exact, and otherwise against the
oracle on the 4096 distinct heads. The input is 4096 seeded heads repeated 4096 times, and every
repetition must give bit-identical results. Outputs start as NaN, so a head that no workgroup wrote
cannot pass.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import exact_tiled_attention_07_amd as fa
from exact_tiled_attention_07_amd.inputs import bf16_bits_to_f32, make_qkv, make_qkv_fp8, to_torch_bf16

from parity import assert_parity, compare

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
FA_MAX_BH = 1 << 24  # include/fa.h
DISTINCT = 4096
REPS = FA_MAX_BH // DISTINCT
D = 64
SCALE = 0.125


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def repeat(t):
    """[1, DISTINCT, 1, D] -> [REPS, DISTINCT, 1, D] on the GPU."""
    return t.to(DEV).repeat(REPS, 1, 1, 1)


def nan_like(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


def same_in_every_repetition(t):
    """All REPS copies bit-identical to the first (compared as integers, so NaN fails)."""
    bits = t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
    return torch.equal(bits, bits[:1].expand_as(bits))


@pytest.fixture(scope="module")
def inputs():
    qb, kb, vb = make_qkv(1, DISTINCT, 1, D, seed=24)
    return qb, kb, vb


def test_fwd_most_heads(inputs):
    qb, kb, vb = inputs
    say(f"[gpu] fa_fwd B*H={FA_MAX_BH} T=1")
    q, k, v = (repeat(to_torch_bf16(x)) for x in (qb, kb, vb))
    o, lse = nan_like(q.shape, torch.bfloat16), nan_like(q.shape[:3], torch.float32)
    fa.fwd(q, k, v, causal=True, scale=SCALE, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), v.view(torch.int16))
    assert same_in_every_repetition(lse)
    o_ref, lse_ref = oracle.attention_fwd(qb, kb, vb, True, SCALE)
    assert_parity(compare(bf16_bits_to_f32(vb), lse[:1].cpu().numpy(), o_ref, lse_ref), "fa_fwd")


def test_sparse_most_heads(inputs):
    qb, kb, vb = inputs
    say(f"[gpu] fa_fwd_sparse B*H={FA_MAX_BH} T=1")
    q, k, v = (repeat(to_torch_bf16(x)) for x in (qb, kb, vb))
    mask = torch.ones(fa.sparse_mask_shape(1, 1), dtype=torch.uint8, device=DEV)
    o, lse = nan_like(q.shape, torch.bfloat16), nan_like(q.shape[:3], torch.float32)
    fa.fwd_sparse(q, k, v, mask, causal=True, scale=SCALE, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), v.view(torch.int16))
    assert same_in_every_repetition(lse)
    _, lse_ref = oracle.attention_fwd(qb, kb, vb, True, SCALE)
    np.testing.assert_allclose(lse[:1].cpu().numpy(), lse_ref, rtol=0, atol=1e-3)


def test_partial_and_splitkv_most_heads(inputs):
    qb, kb, vb = inputs
    say(f"[gpu] fa_fwd_partial and fa_fwd_splitkv B*H={FA_MAX_BH} T=Tk=1")
    q, k, v = (repeat(to_torch_bf16(x)) for x in (qb, kb, vb))
    o_part = nan_like(q.shape, torch.float32)
    lse_part = nan_like(q.shape[:3], torch.float32)
    fa.fwd_partial(q, k, v, 0, 1, causal=True, scale=SCALE, o_part=o_part, lse_part=lse_part)
    torch.cuda.synchronize()
    # fp32 partial O of one key: V divided by the fp32 weight sum l, and that weight is exp2 of the
    # rounding residual of the scaled max (the FMA s * c - m is not rounded), within 2^-23 of 1; the
    # reciprocal and the product add an ulp each
    assert not torch.isnan(o_part).any()
    torch.testing.assert_close(o_part, v.float(), rtol=2.0 ** -21, atol=0.0)
    assert same_in_every_repetition(lse_part)
    _, lse_ref = oracle.attention_fwd(qb, kb, vb, True, SCALE)
    np.testing.assert_allclose(lse_part[:1].cpu().numpy(), lse_ref, rtol=0, atol=1e-3)
    del o_part, lse_part
    o, lse = nan_like(q.shape, torch.bfloat16), nan_like(q.shape[:3], torch.float32)
    fa.fwd_splitkv(q, k, v, causal=True, scale=SCALE, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), v.view(torch.int16))
    assert same_in_every_repetition(lse)
    np.testing.assert_allclose(lse[:1].cpu().numpy(), lse_ref, rtol=0, atol=1e-3)


def test_fp8_most_heads():
    q8, k8, v8, scales = make_qkv_fp8(1, DISTINCT, 1, D, seed=25)
    say(f"[gpu] fa_fwd_fp8 B*H={FA_MAX_BH} T=1")
    q, k, v = (repeat(torch.from_numpy(x)) for x in (q8, k8, v8))
    o, lse = nan_like(q.shape, torch.bfloat16), nan_like(q.shape[:3], torch.float32)
    fa.fwd_fp8(q, k, v, *scales, causal=True, scale=SCALE, out=o, lse=lse)
    torch.cuda.synchronize()
    assert same_in_every_repetition(o) and same_in_every_repetition(lse)
    o_ref, lse_ref = oracle.attention_fwd_fp8(q8, k8, v8, True, SCALE, *scales)
    # one key: O is the dequantized V row rounded once to bf16, so within one bf16 ulp of it
    o1 = o[:1].float().cpu().numpy()
    # (plus the fp32 rounding of the descale product before it)
    assert np.all(np.abs(o1 - o_ref) <= np.abs(o_ref) * (2.0 ** -8 + 2.0 ** -20))
    np.testing.assert_allclose(lse[:1].cpu().numpy(), lse_ref, rtol=0, atol=1e-3)


def test_bwd_most_heads(inputs):
    qb, kb, vb = inputs
    (dob,) = make_qkv(1, DISTINCT, 1, D, seed=26)[:1]
    say(f"[gpu] fa_bwd B*H={FA_MAX_BH} T=1")
    q, k, v, do = (repeat(to_torch_bf16(x)) for x in (qb, kb, vb, dob))
    o, lse = fa.fwd(q, k, v, causal=True, scale=SCALE)
    dq, dk, dv = (nan_like(q.shape, torch.bfloat16) for _ in range(3))
    delta = nan_like(q.shape[:3], torch.float32)
    fa.bwd(q, k, v, o, lse, do, causal=True, scale=SCALE, dq=dq, dk=dk, dv=dv, delta=delta)
    torch.cuda.synchronize()
    # one key: P = 1, so dV = P^T dO = dO exactly, and dS = P (dP - D) = 0 up to the fp32 rounding of
    # dP = dO.V and D = dO.O (each a sum of d products)
    assert torch.equal(dv.view(torch.int16), do.view(torch.int16))
    for t in (dq, dk, delta):
        assert same_in_every_repetition(t)
    qf, kf, vf, dof = (np.abs(bf16_bits_to_f32(x).astype(np.float64)) for x in (qb, kb, vb, dob))
    cancel = D * 2.0 ** -24 * float(dof.sum(axis=-1).max()) * float(vf.max())
    assert float(dq[:1].float().abs().max()) <= 2 * SCALE * float(kf.max()) * cancel
    assert float(dk[:1].float().abs().max()) <= 2 * SCALE * float(qf.max()) * cancel
    _, _, _, delta_ref = oracle.attention_bwd(qb, kb, vb, dob, True, SCALE)
    # D = dO.O in fp32 over d products (O = V exactly here)
    np.testing.assert_allclose(delta[:1].cpu().numpy(), delta_ref, rtol=0, atol=cancel)

"""Randomised parity of every entry point (through the C-ABI) with the CPU oracle (hypothesis,
derandomised so that every run draws the same cases).

- fa_fwd: B, H, T <= 300, d in {64, 128}, causal or not, scale in {1/sqrt(d), 0.01, 1} and an
  input magnitude; every element within the bound derived from the kernel's roundings
  (tests/fwd_bounds.py) and, for sigma <= 1 (the N(0,1) regime it is written for), at the dense
  tolerance;
- fa_bwd: the same ranges plus scale 0.3 and sigma 4, at the backward's tolerance (including its
  allowance for heads dominated by one key);
- fa_fwd_sparse: random masks, one for every head or one per head, empty rows exact;
- fa_fwd_splitkv and fa_fwd_partial: T queries over Tk keys with random split counts and random
  key ranges, against the cross oracle;
- fa_fwd_fp8: against the exact attention of the decoded values within the FP8 bound.
Small shapes, so the whole file takes seconds; the fixed cases of the other files cover the large
ones.
"""
import math

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings, strategies as st

import oracle
import exact_tiled_attention_07_amd as fa
from exact_tiled_attention_07_amd.inputs import make_qkv, make_qkv_fp8, to_torch_bf16

from fwd_bounds import check_bounds, element_bounds
from parity import assert_parity, compare
import test_bwd_parity_gpu as bwd_tests
import test_fp8_parity_gpu as fp8_tests
import test_splitkv_parity_gpu as splitkv_tests

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SETTINGS = settings(max_examples=60, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
FEWER = settings(SETTINGS, max_examples=40)


@SETTINGS
@given(B=st.integers(1, 3), H=st.integers(1, 5), T=st.integers(1, 300), d=st.sampled_from([64, 128]),
       causal=st.booleans(), scale_kind=st.sampled_from(["inv_sqrt_d", "0.01", "1"]),
       sigma=st.sampled_from([0.5, 1.0, 2.0]), seed=st.integers(0, 2 ** 20))
def test_random_shapes_against_oracle(B, H, T, d, causal, scale_kind, sigma, seed):
    scale = {"inv_sqrt_d": 1.0 / math.sqrt(d), "0.01": 0.01, "1": 1.0}[scale_kind]
    qb, kb, vb = make_qkv(B, H, T, d, seed=seed, sigma=sigma)
    print(f"[gpu property] B{B} H{H} T{T} d{d} causal={causal} scale={scale} sigma={sigma} seed={seed}",
          flush=True)
    q, k, v = (to_torch_bf16(x, DEV) for x in (qb, kb, vb))
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd(qb, kb, vb, causal, scale)
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    label = f"B{B} H{H} T{T} d{d} causal={causal} scale={scale} sigma={sigma}"
    if sigma <= 1.0:
        # the stated tolerance is written for N(0,1) inputs. At sigma 2 a non-top weight near 1,
        # rounded to bf16 (2^-9 relative), times a |v| of up to ~8 can exceed it where |O| < 2 (rows
        # with few keys at any scale, or sharp rows at scale 1), so only the derived bound below
        # holds there (the every-row test of the sigma-2 workload C4 still asserts it)
        assert_parity(compare(o, lse, o_ref, lse_ref), label)
    # and every element within the bound derived from the kernel's roundings (tests/fwd_bounds.py)
    ro, rl = check_bounds(o, lse, o_ref, lse_ref, element_bounds(qb, kb, vb, causal, scale))
    assert ro <= 1.0 and rl <= 1.0, (label, ro, rl)


@FEWER
@given(B=st.integers(1, 2), H=st.integers(1, 3), T=st.integers(1, 300), d=st.sampled_from([64, 128]),
       causal=st.booleans(), scale_kind=st.sampled_from(["inv_sqrt_d", "0.01", "0.3", "1"]),
       sigma=st.sampled_from([0.5, 1.0, 2.0, 4.0]), seed=st.integers(0, 2 ** 20))
def test_random_backward(B, H, T, d, causal, scale_kind, sigma, seed):
    scale = {"inv_sqrt_d": 1.0 / math.sqrt(d), "0.01": 0.01, "0.3": 0.3, "1": 1.0}[scale_kind]
    qb, kb, vb = make_qkv(B, H, T, d, seed=seed, sigma=sigma)
    dob, _, _ = make_qkv(B, H, T, d, seed=seed + 1)
    bwd_tests.check(qb, kb, vb, dob, causal, scale, f"property B{B} H{H} T{T} d{d} sigma={sigma}")


@FEWER
@given(H=st.integers(1, 3), T=st.integers(1, 700), d=st.sampled_from([64, 128]), causal=st.booleans(),
       density=st.floats(0.0, 1.0), per_head=st.booleans(), seed=st.integers(0, 2 ** 20))
def test_random_block_sparse(H, T, d, causal, density, per_head, seed):
    qb, kb, vb = make_qkv(1, H, T, d, seed=seed)
    nq, nk = -(-T // 128), -(-T // 64)
    mask = (np.random.default_rng(seed).random((H if per_head else 1, nq, nk)) < density).astype(np.uint8)
    print(f"[gpu property] sparse H{H} T{T} d{d} causal={causal} density={density:.2f} "
          f"per_head={per_head} seed={seed}", flush=True)
    q, k, v = (to_torch_bf16(x, DEV) for x in (qb, kb, vb))
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.fwd_sparse(q, k, v, torch.from_numpy(mask).to(DEV), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    o_ref, lse_ref = oracle.attention_fwd_blockmask(qb, kb, vb, causal, scale, mask, 128, 64)
    empty = np.isneginf(lse_ref)
    np.testing.assert_array_equal(np.isneginf(lse), empty)
    assert np.all(o[empty] == 0.0)
    assert_parity(compare(o[~empty], lse[~empty], o_ref[~empty], lse_ref[~empty]), "property sparse")
    ro, rl = check_bounds(o, lse, o_ref, lse_ref, element_bounds(qb, kb, vb, causal, scale, block_mask=mask))
    assert ro <= 1.0 and rl <= 1.0, (ro, rl)


@FEWER
@given(B=st.integers(1, 2), H=st.integers(1, 3), T=st.integers(1, 200), Tk=st.integers(1, 4000),
       d=st.sampled_from([64, 128]), causal=st.booleans(), n=st.one_of(st.none(), st.integers(1, 40)),
       seed=st.integers(0, 2 ** 20))
def test_random_splitkv(B, H, T, Tk, d, causal, n, seed):
    qb, _, _ = make_qkv(B, H, T, d, seed=seed)
    _, kb, vb = make_qkv(B, H, Tk, d, seed=seed + 1)
    print(f"[gpu property] splitkv B{B} H{H} T{T} Tk{Tk} d{d} causal={causal} n={n} seed={seed}", flush=True)
    q, k, v = (to_torch_bf16(x, DEV) for x in (qb, kb, vb))
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.fwd_splitkv(q, k, v, causal=causal, scale=scale, n_splits=n)
    torch.cuda.synchronize()
    splitkv_tests.check_against_cross(o, lse, oracle.attention_fwd_cross(qb, kb, vb, causal, scale),
                                      "property splitkv")


@FEWER
@given(H=st.integers(1, 3), T=st.integers(1, 200), Tk=st.integers(1, 3000), d=st.sampled_from([64, 128]),
       causal=st.booleans(), a=st.integers(0, 60), b=st.integers(0, 60), seed=st.integers(0, 2 ** 20))
def test_random_partial_ranges(H, T, Tk, d, causal, a, b, seed):
    nt = -(-Tk // 64)  # key ranges start on a 64-key tile and end on one or at Tk
    k_begin = 64 * min(a, nt - 1)
    k_end = max(k_begin, min(Tk, 64 * min(max(a, b) + 1, nt)) if b % 7 else Tk)
    qb, _, _ = make_qkv(1, H, T, d, seed=seed)
    _, kb, vb = make_qkv(1, H, Tk, d, seed=seed + 1)
    print(f"[gpu property] partial H{H} T{T} Tk{Tk} d{d} causal={causal} keys=[{k_begin},{k_end}) "
          f"seed={seed}", flush=True)
    q, k, v = (to_torch_bf16(x, DEV) for x in (qb, kb, vb))
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.fwd_partial(q, k, v, k_begin, k_end, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.attention_fwd_cross(qb, kb, vb, causal, scale, k_begin, k_end)
    splitkv_tests.check_against_cross(o, lse, ref, "property partial")


@FEWER
@given(B=st.integers(1, 2), H=st.integers(1, 3), T=st.integers(1, 600), d=st.sampled_from([64, 128]),
       causal=st.booleans(), scale_kind=st.sampled_from(["inv_sqrt_d", "0.01", "1"]),
       sigma=st.sampled_from([0.5, 1.0, 2.0]), seed=st.integers(0, 2 ** 20))
def test_random_fp8(B, H, T, d, causal, scale_kind, sigma, seed):
    scale = {"inv_sqrt_d": 1.0 / math.sqrt(d), "0.01": 0.01, "1": 1.0}[scale_kind]
    q8, k8, v8, scales = make_qkv_fp8(B, H, T, d, seed=seed, sigma=sigma)
    fp8_tests.check(q8, k8, v8, scales, causal, scale, f"property B{B} H{H} T{T} d{d} sigma={sigma}")

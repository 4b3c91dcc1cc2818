"""Randomised parity of fa_fwd (through the C-ABI) with the CPU oracle (hypothesis, derandomised so
that every run draws the same cases).

Each case draws B, H, T <= 300, d in {64, 128}, causal or not, scale in {1/sqrt(d), 0.01, 1} and an
input magnitude, runs the default launch on the GPU and compares every element with the oracle at
the dense tolerance and within the bound derived from the kernel's roundings (tests/fwd_bounds.py). Small shapes, so the whole file takes seconds; the fixed cases of the other
files cover the large ones.
"""
import math

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings, strategies as st

import oracle
import exact_tiled_attention_07_amd as fa
from exact_tiled_attention_07_amd.inputs import make_qkv, to_torch_bf16

from fwd_bounds import check_bounds, element_bounds
from parity import assert_parity, compare

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SETTINGS = settings(max_examples=60, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])


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
    assert_parity(compare(o, lse, o_ref, lse_ref), label)
    # and every element within the bound derived from the kernel's roundings (tests/fwd_bounds.py)
    ro, rl = check_bounds(o, lse, o_ref, lse_ref, element_bounds(qb, kb, vb, causal, scale))
    assert ro <= 1.0 and rl <= 1.0, (label, ro, rl)

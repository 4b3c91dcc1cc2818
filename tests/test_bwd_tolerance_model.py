"""The backward's GPU tolerance, re-derived on every run (CPU only).

tests/bwd_rounding_model.py applies to the oracle's exact gradients the roundings any bf16 block
algorithm must make (bf16 O and fp32 LSE read back from the forward, bf16 P and dS before the matrix
products, bf16 gradients). Its worst errors over the GPU tests' input cases are stored in
tests/golden/bwd_rounding_model.json by a committed script; this test recomputes them, checks the
stored figures, and checks that the GPU tests' bounds are the stated multiple of them.
"""
import json
import os

import numpy as np
import pytest

import bwd_rounding_model as model
import oracle
from bwd_tolerance import ELEM_TOL, MODEL, RMS_TOL, TOL_FACTOR

HERE = os.path.dirname(os.path.abspath(__file__))


def test_model_figures_match_the_stored_ones():
    fig = model.model_figures()
    stored = json.load(open(os.path.join(HERE, "golden", "bwd_rounding_model.json")))
    assert fig["elem_max"] == pytest.approx(stored["elem_max"], rel=1e-9)
    assert fig["rms_max"] == pytest.approx(stored["rms_max"], rel=1e-9)
    assert fig["elem_where"] == stored["elem_where"] and fig["rms_where"] == stored["rms_where"]


def test_gpu_bounds_are_the_stated_multiple_of_the_model():
    assert ELEM_TOL == pytest.approx(TOL_FACTOR * MODEL["elem_max"])
    assert RMS_TOL == pytest.approx(TOL_FACTOR * MODEL["rms_max"])
    assert 1.5 <= TOL_FACTOR <= 2.5


def test_model_without_roundings_is_the_oracle():
    # the model's float64 arithmetic, with the roundings switched off, agrees with the oracle: the
    # model's error is its roundings and nothing else
    qb, kb, vb, dob = model.inputs(1, 2, 130, 11)
    saved = model.bf16
    try:
        model.bf16 = lambda x: np.asarray(x, dtype=np.float64)
        got = model.model_bwd(qb, kb, vb, dob, True, 0.125)
    finally:
        model.bf16 = saved
    ref = oracle.attention_bwd(qb, kb, vb, dob, True, 0.125)
    for g, r in zip(got[:3], ref[:3]):
        # only the fp32 LSE remains: relative error ~1e-7
        np.testing.assert_allclose(g, r, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("causal", [False, True])
def test_o_rounding_allowance_covers_a_head_dominated_by_one_key(causal):
    # two tokens at scale 1: every row's weights are dominated by one key, dS is a small difference
    # of two large terms everywhere, and dQ, dK are near zero. The rounding model (bf16 O in D, bf16
    # P and dS) then fails the relative bounds, and its excess is what bwd_tolerance's allowance,
    # computed from the same bf16 O, bounds
    from bwd_tolerance import o_rounding_allowance
    from exact_tiled_attention_07_amd.inputs import make_qkv

    qb, kb, vb = make_qkv(1, 1, 2, 64, seed=0)
    dob, _, _ = make_qkv(1, 1, 2, 64, seed=1)
    ref = oracle.attention_bwd(qb, kb, vb, dob, causal, 1.0)
    got = model.model_bwd(qb, kb, vb, dob, causal, 1.0)
    o16 = model.bf16(oracle.attention_fwd(qb, kb, vb, causal, 1.0)[0])
    aq, ak, _ = o_rounding_allowance(qb, kb, vb, dob, causal, 1.0, o16)
    plain = [model.grad_stats(g, r) for g, r in zip(got[:2], ref[:2])]
    if not causal:  # (causal: row 0 sees one key, row 1 two; whichever way, the allowance must cover)
        assert any(s["max_ratio"] > ELEM_TOL or s["rms_ratio"] > RMS_TOL for s in plain)
    for g, r, a in zip(got[:2], ref[:2], (aq, ak)):
        s = model.grad_stats(g, r, 1.1 * a)
        assert s["max_ratio"] <= ELEM_TOL and s["rms_ratio"] <= RMS_TOL, s


def test_o_rounding_allowance_is_small_in_an_ordinary_head():
    # in a head of the tests' usual scale the allowance is a small part of the gradients: it only
    # matters where the relative bounds cannot work
    from bwd_tolerance import o_rounding_allowance

    qb, kb, vb, dob = model.inputs(1, 2, 300, 13)
    ref = oracle.attention_bwd(qb, kb, vb, dob, True, 0.125)
    o16 = model.bf16(oracle.attention_fwd(qb, kb, vb, True, 0.125)[0])
    aq, ak, ad = o_rounding_allowance(qb, kb, vb, dob, True, 0.125, o16)
    assert np.sqrt((aq ** 2).mean()) < 0.02 * np.sqrt((ref[0] ** 2).mean())
    assert np.sqrt((ak ** 2).mean()) < 0.02 * np.sqrt((ref[1] ** 2).mean())
    # and D's allowance bounds the model's D error (the model's D is exactly dO . bf16(O))
    got = model.model_bwd(qb, kb, vb, dob, True, 0.125)
    assert np.all(np.abs(got[3] - ref[3]) <= 1.1 * ad + 1e-6 * np.abs(ref[3]))

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

"""Tolerance of the GPU backward tests, derived from the rounding model (tests/bwd_rounding_model.py).

The stored figures (tests/golden/bwd_rounding_model.json) are the model's worst element error, in
units of |ref| + rms of the head, and its worst rms error, over the GPU tests' input cases. The GPU
may exceed the model by what the model leaves out: fp32 (not fp64) arithmetic for P, dP, D and the
sums, a different summation order, and a forward O within one ulp of the correctly rounded one
rather than equal to it. TOL_FACTOR = 2 allows for that.
"""
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
MODEL = json.load(open(os.path.join(HERE, "golden", "bwd_rounding_model.json")))
TOL_FACTOR = 2.0
ELEM_TOL = TOL_FACTOR * MODEL["elem_max"]   # |gpu - ref| <= ELEM_TOL * (|ref| + rms of the head)
RMS_TOL = TOL_FACTOR * MODEL["rms_max"]     # rms(gpu - ref) <= RMS_TOL * rms(ref), per tensor

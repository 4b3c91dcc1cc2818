"""The FP8 tests' whole-head error bounds against their row-by-row form (CPU).

``fp8_bounds.error_model_heads`` evaluates the bounds of ``error_model_rows`` for every row with
whole-head matrix products; the GPU test of every row of the T = 4096 workload relies on it, so the
two must agree on every row (causal and not, both head dims, a ragged length, unequal descales).
"""
import numpy as np
import pytest

from exact_tiled_attention_07_amd.inputs import make_qkv_fp8
from fp8_bounds import error_model_heads, error_model_rows


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("T,d", [(1, 64), (67, 64), (130, 128)])
def test_heads_equal_rows(T, d, causal):
    q8, k8, v8, scales = make_qkv_fp8(2, 2, T, d, seed=900 + T + d, sigma=2.0)
    scales = (scales[0] * 3, scales[1], scales[2] * 0.5)
    scale = 1.0 / np.sqrt(d)
    rows = [(b, h, i) for b in range(2) for h in range(2) for i in range(T)]
    rb, rl, rp = error_model_rows(q8, k8, v8, scales, causal, scale, rows)
    hb, hl, hp = error_model_heads(q8, k8, v8, scales, causal, scale)
    np.testing.assert_allclose(hb.reshape(-1, d), rb, rtol=1e-9, atol=0)
    np.testing.assert_allclose(hl.reshape(-1), rl, rtol=1e-9, atol=0)
    np.testing.assert_allclose(hp.reshape(-1, d), rp, rtol=1e-9, atol=0)


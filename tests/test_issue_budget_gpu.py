"""Issue rates of the forward's inner-loop instructions on the device (tests/issue_rate_probe.hip),
the measured basis of the d = 64 forward's per-tile cycle budget.

Per SIMD, in cycles, with the SIMD's own elapsed time (its slowest wave): the MFMA 32x32x16 bf16
takes 32 cycles at every occupancy; v_exp_f32 issues at about a third of the rate of v_fma_f32; and
the softmax's minimal instruction mix for one 64-key tile at d = 64 (about 9 VALU instructions per
MFMA) keeps the SIMD busy well beyond the MFMA time, more so with the fragment reads from LDS. The
MFMAs do not hide wholly behind the VALU work of the other waves: each one adds to the time of the
mix alone, more for two 16x16x32 instructions than for one 32x32x16 of the same flops, and the same
with the accumulators in AGPRs. The FP8 forward's conversion of its weights, v_cvt_pk_fp8_f32,
issues at the rate of v_exp_f32. These are the facts the kernels' design notes rely on; the test
asserts them loosely and prints the table.
"""
import ctypes
import os

import pytest

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libissue_rate_probe.so")
ITERS = 2000
MODES = {0: "16 fma", 1: "16 exp", 2: "16 add", 3: "16 max3", 4: "16 cvt_pk_bf16", 5: "4 mfma",
         6: "4 mfma + softmax mix (37 VALU)", 7: "mode 6 + 6 LDS reads", 8: "mode 6 + 3 LDS reads",
         9: "two roles: 4 mfma | 37 VALU", 10: "the 37 VALU alone", 11: "16 cvt_pk_fp8",
         12: "2 fp8 mfma (128 cycles) + 37 VALU", 13: "8 mfma 16x16x32 + 37 VALU",
         14: "mode 6, accumulators in AGPRs", 15: "2 fp8 mfma 32x32x64"}


@pytest.fixture(scope="module")
def cycles():
    assert os.path.exists(PROBE), f"{PROBE} is not built (__graft_entry__.build())"
    lib = ctypes.CDLL(PROBE)
    lib.issue_rate_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.POINTER(ctypes.c_double)]
    lib.issue_rate_probe.restype = ctypes.c_int
    out = {}
    for w in (1, 2, 3, 4):
        for m in MODES:
            if m == 9 and w % 2:
                continue
            c = ctypes.c_double()
            assert lib.issue_rate_probe(m, w, ITERS, ctypes.byref(c)) == 0
            # cycles per SIMD for one unit of the mode's work (one wave's iteration; mode 9 splits
            # one unit over two waves)
            units = w if m != 9 else w // 2
            out[(m, w)] = c.value / ITERS / units
    for (m, w), v in sorted(out.items(), key=lambda kv: (kv[0][1], kv[0][0])):
        print(f"[gpu issue] waves/SIMD {w}  {MODES[m]:32s} {v:8.1f} cycles per unit", flush=True)
    return out


def test_mfma_takes_32_cycles_at_every_occupancy(cycles):
    for w in (1, 2, 3, 4):
        assert cycles[(5, w)] == pytest.approx(128.0, rel=0.03)


def test_exp_is_several_times_slower_than_fma(cycles):
    assert cycles[(1, 4)] > 2.5 * cycles[(0, 4)]
    # one wave alone issues VALU work far slower than several waves together
    assert cycles[(0, 1)] > 2.0 * cycles[(0, 4)]


def test_softmax_mix_caps_the_mfma(cycles):
    for w in (3, 4):
        # the minimal softmax work per 4 MFMAs keeps the SIMD busy at least 1.4x the MFMA time ...
        assert cycles[(6, w)] > 1.4 * 128.0
        # ... and the fragment reads of one 32-query wave add to it
        assert cycles[(7, w)] > cycles[(6, w)]
    # splitting the same work into MFMA-only and VALU-only waves is not faster
    assert cycles[(9, 4)] > cycles[(6, 4)]


def test_mfma_adds_to_the_mix(cycles):
    for w in (3, 4):
        # the mix alone takes longer than its 4 MFMAs, and the MFMAs still add to it
        assert cycles[(10, w)] > 128.0
        assert cycles[(6, w)] > cycles[(10, w)] + 4 * 5.0
        # the same flops in twice the instructions (16x16x32) cost more ...
        assert cycles[(13, w)] > cycles[(6, w)]
        # ... and the same 128 MFMA cycles in half the instructions (FP8 32x32x64) no more
        assert cycles[(12, w)] < cycles[(6, w)] * 1.03
        # accumulators in AGPRs instead of VGPRs change nothing for the better
        assert cycles[(14, w)] > cycles[(6, w)] * 0.97


def test_fp8_conversion_issues_like_exp(cycles):
    assert cycles[(15, 4)] == pytest.approx(128.0, rel=0.03)  # 64 cycles per FP8 32x32x64
    assert cycles[(11, 4)] > 1.5 * cycles[(4, 4)]
    assert cycles[(11, 4)] == pytest.approx(cycles[(1, 4)], rel=0.2)

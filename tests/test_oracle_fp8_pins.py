"""Pins of the FP8 oracle and of the FP8 input generator (CPU).

F1 the E4M3 decode equals torch's float8_e4m3fn conversion for all 256 codes.
F2 closed forms of the format: 1, 448, the smallest normal and subnormal, -0, NaN.
F3 with descales of 1 the FP8 oracle equals the dense bf16 oracle on the same values bit for bit
   (every E4M3 value is a bf16 value).
F4 power-of-two descales: q and k descales act as a factor on the scale, the v descale as a factor on
   O only (exact identities in binary floating point).
F5 the generator's quantization: round to nearest (the nearest code, found by brute force over the
   decoded table, with ties to the even code), amax maps to 448, per-tensor descale amax / 448.
F6 the row entry for long heads (numpy) equals the whole-head FP8 oracle on every row.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_07_amd.inputs import bf16_bits_from_f32, make_qkv_fp8, quantize_e4m3


def test_f1_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])


def test_f2_closed_forms():
    d = oracle.e4m3_to_f64(np.array([0x38, 0x7E, 0x08, 0x01, 0x80, 0x7F, 0xFF, 0xB8, 0x3C], np.uint8))
    assert d[0] == 1.0 and d[1] == 448.0 and d[2] == 2.0 ** -6 and d[3] == 2.0 ** -9
    assert d[4] == 0.0 and np.signbit(d[4]) and np.isnan(d[5]) and np.isnan(d[6])
    assert d[7] == -1.0 and d[8] == 1.5


@pytest.mark.parametrize("causal", [True, False])
def test_f3_unit_descale_is_the_bf16_oracle(causal):
    q8, k8, v8, _ = make_qkv_fp8(2, 2, 130, 64, seed=3)
    o8, l8 = oracle.attention_fwd_fp8(q8, k8, v8, causal, 0.125, 1.0, 1.0, 1.0)
    bits = [bf16_bits_from_f32(oracle.e4m3_to_f64(x).astype(np.float32)) for x in (q8, k8, v8)]
    o, l = oracle.attention_fwd(*bits, causal, 0.125)
    np.testing.assert_array_equal(o8, o)
    np.testing.assert_array_equal(l8, l)


@pytest.mark.parametrize("causal", [True, False])
def test_f4_power_of_two_descales(causal):
    q8, k8, v8, _ = make_qkv_fp8(1, 3, 77, 64, seed=4)
    o1, l1 = oracle.attention_fwd_fp8(q8, k8, v8, causal, 0.125, 1.0, 1.0, 1.0)
    o2, l2 = oracle.attention_fwd_fp8(q8, k8, v8, causal, 0.125 * 2.0 ** -5, 4.0, 8.0, 1.0)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    o3, l3 = oracle.attention_fwd_fp8(q8, k8, v8, causal, 0.125, 1.0, 1.0, 2.0 ** -3)
    np.testing.assert_array_equal(o3, o1 * 2.0 ** -3)
    np.testing.assert_array_equal(l3, l1)


def test_f5_quantization_is_round_to_nearest():
    table = oracle.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    finite = np.where(~np.isnan(table))[0]
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(3000) * 40, (table[finite][1:] + table[finite][:-1]) / 2,
                        [447.9, 448.0, 460.0, -1e4, 2.0 ** -11]]).astype(np.float32)
    got = quantize_e4m3(x, 1.0)
    for xi, gi in zip(x.astype(np.float64), got):
        xc = min(max(xi, -448.0), 448.0)
        dist = np.abs(table[finite] - xc)
        best = finite[dist == dist.min()]
        if len(best) > 1:  # a tie: the even code (ties of +0/-0 at zero aside)
            best = best[(best & 1) == 0]
        assert table[gi] == table[best[0]], (xi, gi, best)
    q8, k8, v8, scales = make_qkv_fp8(1, 2, 50, 64, seed=6)
    for c, s in zip((q8, k8, v8), scales):
        assert np.abs(oracle.e4m3_to_f64(c)).max() == 448.0
        assert s == float(np.float32(s))


@pytest.mark.parametrize("causal", [True, False])
def test_f6_row_entry_matches_the_whole_head_oracle(causal):
    # attention_fwd_fp8_rows (numpy, rows) against attention_fwd_fp8 (the C float64 forward on the
    # decoded values, pinned by F1-F5) on every row of small heads
    q8, k8, v8, sc = make_qkv_fp8(2, 2, 150, 64, seed=71, sigma=2.0)
    o, lse = oracle.attention_fwd_fp8(q8, k8, v8, causal, 0.125, *sc)
    rows = [(b, h, i) for b in range(2) for h in range(2) for i in range(150)]
    ro, rl = oracle.attention_fwd_fp8_rows(q8, k8, v8, causal, 0.125, *sc, rows)
    np.testing.assert_allclose(ro, o.reshape(-1, 64), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(rl, lse.reshape(-1), rtol=1e-12, atol=1e-12)

"""Pins of the CPU block-sparse oracle against facts that do not come from it.

S1 an all-ones block mask is the dense attention (bit for bit against the pinned dense oracle).
S2 a block-diagonal mask is independent attention on each diagonal block (dense oracle on slices).
S3 with 1 x 1 blocks the block mask is an element mask: the lower triangle without the causal flag
   is the causal attention.
S4 rows whose blocks are all masked get O = 0 and LSE = -inf (the reading for an empty softmax).
S5 one allowed key block: scipy's softmax / logsumexp over exactly those keys.
S6 one mask per head equals the shared-mask result head by head.
"""
import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
from exact_tiled_attention_07_amd.inputs import bf16_bits_to_f32, make_qkv


def ones_mask(T, bm, bn, heads=1):
    return np.ones((heads, -(-T // bm), -(-T // bn)), dtype=np.uint8)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("T", [1, 63, 130])
def test_s1_all_ones_is_dense(T, causal):
    q, k, v = make_qkv(2, 2, T, 16, seed=T)
    o, l = oracle.attention_fwd_blockmask(q, k, v, causal, 0.25, ones_mask(T, 128, 64), 128, 64)
    o_d, l_d = oracle.attention_fwd(q, k, v, causal, 0.25)
    np.testing.assert_array_equal(o, o_d)
    np.testing.assert_array_equal(l, l_d)


@pytest.mark.parametrize("causal", [True, False])
def test_s2_block_diagonal_is_independent_blocks(causal):
    T, blk = 200, 64
    q, k, v = make_qkv(1, 3, T, 16, seed=5)
    n = -(-T // blk)
    mask = np.eye(n, dtype=np.uint8)[None]
    o, l = oracle.attention_fwd_blockmask(q, k, v, causal, 0.3, mask, blk, blk)
    for b in range(n):
        sl = slice(b * blk, min(T, (b + 1) * blk))
        o_b, l_b = oracle.attention_fwd(q[:, :, sl].copy(), k[:, :, sl].copy(), v[:, :, sl].copy(), causal, 0.3)
        np.testing.assert_array_equal(o[:, :, sl], o_b)
        np.testing.assert_array_equal(l[:, :, sl], l_b)


def test_s3_unit_blocks_make_an_element_mask():
    T = 37
    q, k, v = make_qkv(1, 2, T, 8, seed=9)
    tril = np.tril(np.ones((T, T), dtype=np.uint8))[None]
    o, l = oracle.attention_fwd_blockmask(q, k, v, False, 0.5, tril, 1, 1)
    o_c, l_c = oracle.attention_fwd(q, k, v, True, 0.5)
    np.testing.assert_array_equal(o, o_c)
    np.testing.assert_array_equal(l, l_c)


def test_s4_empty_rows():
    T = 150
    q, k, v = make_qkv(1, 1, T, 16, seed=3)
    mask = ones_mask(T, 64, 64)
    mask[0, 1, :] = 0  # query block 1 (rows 64..127) sees nothing
    for causal in (True, False):
        o, l = oracle.attention_fwd_blockmask(q, k, v, causal, 0.25, mask, 64, 64)
        assert np.all(o[0, 0, 64:128] == 0.0) and np.all(np.isneginf(l[0, 0, 64:128]))
        assert np.all(np.isfinite(l[0, 0, :64])) and np.all(np.isfinite(l[0, 0, 128:]))
    # causal with only key block 1 allowed: rows 0..63 see no key at or before them
    mask = np.zeros_like(mask)
    mask[0, :, 1] = 1
    o, l = oracle.attention_fwd_blockmask(q, k, v, True, 0.25, mask, 64, 64)
    assert np.all(np.isneginf(l[0, 0, :64])) and np.all(np.isfinite(l[0, 0, 64:]))


@pytest.mark.parametrize("causal", [True, False])
def test_s5_one_key_block_against_scipy(causal):
    T, bm, bn, scale = 160, 64, 32, 0.2  # query and key blocks of different sizes
    q, k, v = make_qkv(1, 1, T, 16, seed=11)
    mask = np.zeros((1, -(-T // bm), T // bn), dtype=np.uint8)
    mask[0, :, 2] = 1  # keys 64..95 only
    o, l = oracle.attention_fwd_blockmask(q, k, v, causal, scale, mask, bm, bn)
    qf, kf, vf = (bf16_bits_to_f32(x)[0, 0].astype(np.float64) for x in (q, k, v))
    s = scale * qf @ kf.T
    keys = np.arange(64, 96)
    for i in range(T):
        vis = keys[keys <= i] if causal else keys
        if vis.size == 0:
            assert np.isneginf(l[0, 0, i]) and np.all(o[0, 0, i] == 0)
            continue
        np.testing.assert_allclose(o[0, 0, i], softmax(s[i, vis]) @ vf[vis], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(l[0, 0, i], logsumexp(s[i, vis]), rtol=1e-13)


def test_s6_per_head_masks():
    T, B, H = 130, 2, 2
    q, k, v = make_qkv(B, H, T, 16, seed=13)
    rng = np.random.default_rng(0)
    masks = (rng.random((B * H, -(-T // 64), -(-T // 32))) < 0.5).astype(np.uint8)
    o, l = oracle.attention_fwd_blockmask(q, k, v, False, 0.25, masks, 64, 32)
    for hh in range(B * H):
        b, h = divmod(hh, H)
        o1, l1 = oracle.attention_fwd_blockmask(q, k, v, False, 0.25, masks[hh:hh + 1], 64, 32)
        np.testing.assert_array_equal(o[b, h], o1[b, h])
        np.testing.assert_array_equal(l[b, h], l1[b, h])


def test_mask_shape_checked():
    q, k, v = make_qkv(1, 1, 100, 16, seed=1)
    with pytest.raises(ValueError):
        oracle.attention_fwd_blockmask(q, k, v, True, 0.25, np.ones((1, 1, 1), np.uint8), 64, 64)
    with pytest.raises(ValueError):
        oracle.attention_fwd_blockmask(q, k, v, True, 0.25, np.ones((3, 2, 2), np.uint8), 64, 64)

"""The seeded input generator: bf16 rounding and determinism (no attention arithmetic here)."""
import numpy as np
import torch

from exact_tiled_attention_07_amd.inputs import (WORKLOADS, bf16_bits_from_f32, bf16_bits_to_f32,
                                                 make_qkv, to_torch_bf16, sparse_mask)


def test_rne_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10,
        # exact ties between two bf16 values: the lower 16 bits are 0x8000
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 1e-40, -1e-40], dtype=np.float32),
    ])
    ours = bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    nan = bf16_bits_from_f32(np.array([np.nan], dtype=np.float32))
    assert np.isnan(bf16_bits_to_f32(nan)[0])


def test_roundtrip_and_torch_view():
    b = bf16_bits_from_f32(np.linspace(-5, 5, 1001, dtype=np.float32))
    f = bf16_bits_to_f32(b)
    np.testing.assert_array_equal(bf16_bits_from_f32(f), b)
    t = to_torch_bf16(b)
    assert t.dtype == torch.bfloat16
    np.testing.assert_array_equal(t.float().numpy(), f)


def test_seeded_and_ordered():
    q1, k1, v1 = make_qkv(1, 2, 8, 64, seed=3)
    q2, k2, v2 = make_qkv(1, 2, 8, 64, seed=3)
    assert np.array_equal(q1, q2) and np.array_equal(k1, k2) and np.array_equal(v1, v2)
    assert not np.array_equal(q1, k1) and not np.array_equal(k1, v1)
    g = np.random.Generator(np.random.PCG64(3))
    expect_q = bf16_bits_from_f32(g.standard_normal((1, 2, 8, 64), dtype=np.float32))
    assert np.array_equal(q1, expect_q)
    q4, _, _ = make_qkv(1, 2, 8, 64, seed=3, sigma=2.0)
    np.testing.assert_array_equal(bf16_bits_to_f32(q4), 2 * bf16_bits_to_f32(q1))


def test_workload_table():
    assert WORKLOADS["c4"].sigma == 2.0 and WORKLOADS["c4"].T == 4096
    assert WORKLOADS["c5b"].causal is False and WORKLOADS["c5b"].d == 128
    w = WORKLOADS["c3"]
    assert w.flops == 2.0 * 4 * 12 * 1024 * 1024 * 64
    assert abs(WORKLOADS["c5b"].flops - 4.0 * 4 * 16 * 8192 ** 2 * 128) < 1


def test_sparse_mask():
    # the block-sparse workload's mask: one mask for every head, 128 x 64 blocks, the two diagonal
    # blocks of every query block set, the rest kept at the given density, the same for a seed
    m = sparse_mask(16384, 0.25, 5)
    assert m.shape == (1, 128, 256) and m.dtype == np.uint8 and set(np.unique(m)) <= {0, 1}
    for i in range(128):
        assert m[0, i, 2 * i] == 1 and m[0, i, 2 * i + 1] == 1
    assert 0.24 < m.mean() < 0.27
    np.testing.assert_array_equal(m, sparse_mask(16384, 0.25, 5))
    assert not np.array_equal(m, sparse_mask(16384, 0.25, 6))
    # a ragged length: the last query block's diagonal ends at the last key block
    r = sparse_mask(1000, 0.0, 1)
    assert r.shape == (1, 8, 16) and r[0, 7, 14] == 1 and r[0, 7, 15] == 1 and r.sum() == 16

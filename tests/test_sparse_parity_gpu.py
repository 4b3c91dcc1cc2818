"""Parity of the block-sparse forward (fa_fwd_sparse, through the C-ABI) with the CPU oracle.

Same tolerance as the dense forward (tests/parity.py), applied to the rows that see at least one key;
rows that see none must be exactly O = 0 and LSE = -inf. With an all-ones mask the sparse kernel
visits the same tiles in the same order as the dense one, so its result must equal fa_fwd's bit for
bit.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import exact_tiled_attention_07_amd as fa
from exact_tiled_attention_07_amd.inputs import WORKLOADS, make_qkv, sparse_mask, to_torch_bf16

from fwd_bounds import check_bounds, element_bounds
from parity import assert_parity, assert_rms, compare

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)


def random_mask(T, heads, density, seed):
    nq, nk = -(-T // 128), -(-T // 64)
    return (np.random.default_rng(seed).random((heads, nq, nk)) < density).astype(np.uint8)


def run_sparse(qb, kb, vb, mask, causal, scale):
    q, k, v = (to_torch_bf16(x, DEV) for x in (qb, kb, vb))
    m = torch.from_numpy(mask).to(DEV)
    o, lse = fa.fwd_sparse(q, k, v, m, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check(qb, kb, vb, mask, causal, scale, label, rms=False):
    say(f"[gpu sparse] {label} shape={qb.shape} causal={causal} mask={mask.shape} density={mask.mean():.2f}")
    o, lse = run_sparse(qb, kb, vb, mask, causal, scale)
    o_ref, lse_ref = oracle.attention_fwd_blockmask(qb, kb, vb, causal, scale, mask, 128, 64)
    empty = np.isneginf(lse_ref)
    np.testing.assert_array_equal(np.isneginf(lse), empty)
    assert np.all(o[empty] == 0.0)
    live = ~empty
    stats = compare(o[live], lse[live], o_ref[live], lse_ref[live])
    say(f"[gpu sparse] {label} {stats} empty rows {int(empty.sum())}")
    assert_parity(stats, label)
    if rms:  # i.i.d. zero-mean V over many rows: the relative RMS check too
        assert_rms(stats, label)
    if qb.shape[2] <= 4096:  # and the bound derived from the kernel's roundings (T x T matrices)
        ro, rl = check_bounds(o, lse, o_ref, lse_ref, element_bounds(qb, kb, vb, causal, scale, block_mask=mask))
        say(f"[gpu sparse] {label} derived bound: worst |dO| at {ro:.3f} of it, |dLSE| at {rl:.3f}")
        assert ro <= 1.0 and rl <= 1.0, (label, ro, rl)
    return o, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("T,density", [(1, 1.0), (65, 0.5), (200, 0.5), (1000, 0.3), (2049, 0.6)])
def test_sparse_random_masks(T, density, causal, d):
    qb, kb, vb = make_qkv(1, 3, T, d, seed=3000 + T + d)
    check(qb, kb, vb, random_mask(T, 1, density, T), causal, 1.0 / math.sqrt(d), f"T={T} d={d}")


@pytest.mark.parametrize("causal", [True, False])
def test_sparse_per_head_masks_and_empty_rows(causal):
    B, H, T = 2, 3, 777
    qb, kb, vb = make_qkv(B, H, T, 64, seed=17)
    mask = random_mask(T, B * H, 0.4, 5)
    mask[0, 2, :] = 0          # head 0, query block 2: no key at all
    mask[3, :, 0] = 0          # head 3: key block 0 hidden, so causal rows 0..63 see nothing
    mask[3, 0, 1:] = 1
    check(qb, kb, vb, mask, causal, 0.125, "per-head masks")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_sparse_all_ones_equals_dense(causal, d):
    qb, kb, vb = make_qkv(2, 2, 1000, d, seed=23)
    q, k, v = (to_torch_bf16(x, DEV) for x in (qb, kb, vb))
    ones = torch.ones(fa.sparse_mask_shape(1000, 1), dtype=torch.uint8, device=DEV)
    o_s, l_s = fa.fwd_sparse(q, k, v, ones, causal=causal)
    # the dense forward with the same 128 x 64 tiles (fa_fwd itself takes the key split at this size)
    o_d, l_d = fa.fwd_ex(q, k, v, 128, 64, 4, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o_s.view(torch.int16), o_d.view(torch.int16))
    assert torch.equal(l_s, l_d)


def test_sparse_long_sequence():
    # T = 16384 at 25% of the blocks plus the diagonal ones (every row sees a key), one head
    T = 16384
    qb, kb, vb = make_qkv(1, 1, T, 64, seed=29)
    mask = random_mask(T, 1, 0.25, 7)
    for i in range(mask.shape[1]):
        mask[0, i, 2 * i:2 * i + 2] = 1
    check(qb, kb, vb, mask, True, 0.125, "T=16384")


def test_sparse_bench_workload_every_row():
    # the block-sparse forward as the bench times it: all 48 heads of the causal T = 16384 workload
    # with its mask (25% of the 128 x 64 blocks plus the diagonal ones, seed 5), every row
    wl = WORKLOADS["c5a"]
    qb, kb, vb = wl.make()
    check(qb, kb, vb, sparse_mask(wl.T, 0.25, wl.seed), wl.causal, wl.scale, wl.name + " sparse 25%", rms=True)


def test_sparse_head_groups():
    # B4 H16 T16384 causal: each XCD's 8 heads run 4 at a time (the K/V budget of causal launches);
    # one mask for every head, 25% of the blocks plus the diagonal ones. Every row is written (the
    # outputs start as NaN), and whole heads on both sides of each group boundary match the oracle
    B, H, T, d = 4, 16, 16384, 64
    assert fa.plan(B, H, T, d, True)["head_group"] == 4
    BH = B * H
    qb, kb, vb = make_qkv(B, H, T, d, seed=37)
    mask = random_mask(T, 1, 0.25, 11)
    for i in range(mask.shape[1]):
        mask[0, i, 2 * i:2 * i + 2] = 1
    say(f"[gpu sparse] head groups B{B} H{H} T{T}")
    q, k, v = (to_torch_bf16(x, DEV) for x in (qb, kb, vb))
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, T), float("nan"), dtype=torch.float32, device=DEV)
    fa.fwd_sparse(q, k, v, torch.from_numpy(mask).to(DEV), causal=True, scale=0.125, out=o, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any().item() and not torch.isnan(lse).any().item()
    for bh in (0, 31, 32, 63):  # heads 0..31 form the first group of every XCD, 32..63 the second
        sel = [x.reshape(1, BH, T, d)[:, bh:bh + 1] for x in (qb, kb, vb)]
        o_ref, lse_ref = oracle.attention_fwd_blockmask(*sel, True, 0.125, mask, 128, 64)
        o_g = o.view(BH, T, d)[bh:bh + 1].float().cpu().numpy().astype(np.float64).reshape(1, 1, T, d)
        lse_g = lse.view(BH, T)[bh:bh + 1].cpu().numpy().astype(np.float64).reshape(1, 1, T)
        stats = compare(o_g, lse_g, o_ref, lse_ref)
        say(f"[gpu sparse] head groups, head {bh}: {stats}")
        assert_parity(stats, f"sparse head groups, head {bh}")


def test_sparse_longest_sequence_full_tile_list():
    # FA_SPARSE_MAX_T = 65536, non-causal: 5% of the blocks plus the diagonal ones, and the first and
    # last query blocks with every key block set, so their tile lists hold the 1024 tiles a list
    # can take (T / 64); one head
    T = 65536
    qb, kb, vb = make_qkv(1, 1, T, 64, seed=31)
    mask = random_mask(T, 1, 0.05, 9)
    for i in range(mask.shape[1]):
        mask[0, i, 2 * i:2 * i + 2] = 1
    mask[0, 0, :] = 1
    mask[0, -1, :] = 1
    assert mask.shape == (1, 512, 1024)
    check(qb, kb, vb, mask, False, 0.125, "T=65536 full lists")


def test_sparse_binding_rejects():
    q = torch.zeros(1, 1, 100, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        fa.fwd_sparse(q, q, q, torch.ones((1, 1, 1), dtype=torch.uint8, device=DEV))
    with pytest.raises(TypeError):
        fa.fwd_sparse(q, q, q, torch.ones(fa.sparse_mask_shape(100), dtype=torch.int32, device=DEV))

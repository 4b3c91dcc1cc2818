"""C-ABI of libfa.so on the host: symbols, argument checks, plans. No kernel is ever launched here.

Every call below either fails validation or is an empty problem, and both return before any HIP
call, so these run without a GPU.
"""
import ctypes
import json
import os

import numpy as np
import pytest

from exact_tiled_attention_07_amd import fa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")
A = 0x10000  # fake, 16-byte-aligned, non-overlapping "device" addresses; never dereferenced


def call(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, B=1, H=1, T=8, d=64, causal=1, scale=0.125):
    return fa.lib().fa_fwd(q, k, v, o, lse, B, H, T, d, causal, scale, None)


def test_library_exports_every_declared_function():
    names = fa.header_functions()
    assert names == ["fa_bwd", "fa_fwd", "fa_fwd_ex", "fa_fwd_fp8", "fa_fwd_partial", "fa_fwd_plan",
                     "fa_fwd_sparse", "fa_fwd_splitkv", "fa_fwd_splitkv_noalloc", "fa_merge",
                     "fa_splitkv_splits", "fa_splitkv_workspace_bytes", "fa_strerror"]
    lib = fa.lib()
    for n in names:
        assert hasattr(lib, n)


def test_int_arguments_out_of_c_range_raise():
    # ctypes would wrap 2**32 + 8 to 8 (a valid size) without this check in the binding
    import ctypes
    for kw in ("B", "H", "T"):
        with pytest.raises(ctypes.ArgumentError):
            call(**{kw: (1 << 32) + 8})
    with pytest.raises(ctypes.ArgumentError):
        fa.lib().fa_splitkv_workspace_bytes(1, 1, 8, 64, -(1 << 31) - 1)
    assert call(T=(1 << 31) - 1) == fa.FA_ERR_INVALID_ARG  # in range: the library's own check


def test_null_pointers():
    for kw in ("q", "k", "v", "o", "lse"):
        assert call(**{kw: None}) == fa.FA_ERR_NULL


@pytest.mark.parametrize("kw,val", [("B", -1), ("H", -1), ("T", -1), ("T", (1 << 22) + 1)])
def test_bad_sizes(kw, val):
    assert call(**{kw: val}) == fa.FA_ERR_INVALID_ARG


def test_too_many_heads():
    assert call(B=1 << 13, H=1 << 12) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("d", [0, 16, 32, 63, 65, 96, 256])
def test_unsupported_head_dim(d):
    assert call(d=d) == fa.FA_ERR_UNSUPPORTED_D


@pytest.mark.parametrize("scale", [0.0, -0.125, float("inf"), float("nan"), 3.0e38])
def test_bad_scale(scale):
    # 3e38 is a finite fp32 whose product with log2(e), the factor the kernels use, is not
    assert call(scale=scale) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,val", [("q", A + 8), ("k", 2 * A + 2), ("v", 3 * A + 4), ("o", 4 * A + 1),
                                    ("lse", 5 * A + 2)])
def test_misaligned(kw, val):
    assert call(**{kw: val}) == fa.FA_ERR_ALIGNMENT


def test_lse_only_needs_4_bytes():
    # passes every check and is empty (T=0), so nothing is launched
    assert call(lse=5 * A + 4, T=0) == fa.FA_OK


@pytest.mark.parametrize("o,lse", [(A, 5 * A), (A + 512, 5 * A), (4 * A, 3 * A + 16), (4 * A, 4 * A + 64)])
def test_overlapping_outputs(o, lse):
    # q/k/v occupy [A, A+1024), ... with T=8, d=64 (1 KiB each)
    assert call(o=o, lse=lse) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("shape", [(0, 3, 8, 64), (2, 0, 8, 64), (2, 3, 0, 128)])
def test_empty_problem_is_ok(shape):
    B, H, T, d = shape
    assert call(B=B, H=H, T=T, d=d) == fa.FA_OK
    assert call(B=B, H=H, T=T, d=d, causal=0) == fa.FA_OK


def test_fwd_ex_tile_checks():
    L = fa.lib()
    args = (A, 2 * A, 3 * A, 4 * A, 5 * A, 1, 1, 0, 64, 1, 0.125, None)
    assert L.fa_fwd_ex(*args, 0, 0, 0) == fa.FA_ERR_TILE        # must force a shape
    assert L.fa_fwd_ex(*args, 96, 64, 3) == fa.FA_ERR_TILE       # not in the table
    assert L.fa_fwd_ex(*args, 64, 64, -2) == fa.FA_ERR_TILE
    assert L.fa_fwd_ex(*args, 64, 64, 2) == fa.FA_OK             # supported, empty problem
    args128 = (A, 2 * A, 3 * A, 4 * A, 5 * A, 1, 1, 0, 128, 1, 0.125, None)
    assert L.fa_fwd_ex(*args128, 128, 64, 4) == fa.FA_OK


def test_strerror_covers_codes():
    seen = set()
    for code in range(-7, 1):
        s = fa.strerror(code)
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 8
    assert fa.strerror(-99) == "unknown status"


def test_plan_matches_the_pages_launch_count():
    fact = json.load(open(GOLDEN))["programs_T4096"]
    p = fa.plan(fact["B"], fact["H"], fact["T"], 64, True, fact["block_m"], fact["block_n"], 2)
    assert p["grid"] == fact["programs"] == 3072
    assert p["q_blocks"] == 64


def test_plan_default_and_tile_counts():
    p = fa.plan(4, 12, 4096, 64, True)
    assert p["block_m"] % (32 * p["waves"]) == 0
    nq = -(-4096 // p["block_m"])
    assert p["q_blocks"] == nq and p["grid"] == nq * 48
    # causal: Q block i needs ceil(min((i+1)*BM, T) / BN) tiles
    bm, bn = p["block_m"], p["block_n"]
    expect = sum(-(-min((i + 1) * bm, 4096) // bn) for i in range(nq)) * 48
    assert p["kv_tiles"] == expect
    full = fa.plan(4, 16, 8192, 128, False)
    assert full["kv_tiles"] == full["grid"] * (-(-8192 // full["block_n"]))
    assert full["lds_bytes"] == 4 * full["block_n"] * 128 * 2
    ragged = fa.plan(2, 12, 1000, 64, True)
    assert ragged["q_blocks"] == -(-1000 // ragged["block_m"])
    assert fa.plan(0, 12, 1000, 64, True)["grid"] == 0


def test_plan_default_tile_for_short_sequences():
    # d = 64 picks among the key split, 128-key tiles and the 128 x 64 default by the grid of the
    # 128 x 64 launch (nq = ceil(T/128) Q blocks per head, grid = nq*B*H)
    def pick(B, H, T, causal):
        p = fa.plan(B, H, T, 64, causal)
        return "split" if p["key_split"] == 2 else f"{p['block_m']}x{p['block_n']}"
    ks = fa.plan(3, 12, 1024, 64, True)  # nq 8, grid 288: the key split
    assert (ks["key_split"], ks["block_m"], ks["waves"], ks["lds_bytes"]) == (2, 64, 4, 65536)
    assert ks["grid"] == 16 * 36
    assert pick(2, 12, 1000, True) == "split"     # nq 8, grid 192
    assert pick(1, 12, 4096, True) == "split"     # nq 32, grid 384
    assert pick(4, 12, 1024, True) == "128x128"   # nq 8, grid 384
    assert pick(16, 12, 1024, True) == "128x128"  # nq 8, grid 1536
    assert pick(4, 12, 2048, True) == "128x128"   # nq 16, grid 768
    assert pick(8, 12, 2048, True) == "128x64"    # nq 16, grid 1536
    assert pick(4, 12, 4096, True) == "128x64"    # nq 32, grid 1536
    assert pick(4, 12, 512, True) == "128x64"     # nq 4
    assert pick(1, 12, 1024, False) == "split"    # non-causal, grid 96
    assert pick(4, 12, 1024, False) == "128x128"  # non-causal, grid 384
    assert pick(4, 16, 8192, False) == "128x64"   # non-causal, grid 4096
    assert fa.plan(1, 1, 8, 128, True)["key_split"] == 1      # d = 128: 128 x 64 ...
    assert fa.plan(1, 1, 8, 128, True)["block_n"] == 64
    assert fa.plan(4, 16, 8192, 128, True)["block_m"] == 128
    p = fa.plan(4, 16, 8192, 128, False)                        # ... or, non-causal from T = 2048,
    assert (p["block_m"], p["block_n"], p["waves"], p["grid"]) == (256, 64, 8, 32 * 64)  # 256 x 64 x 8
    assert fa.plan(4, 16, 1024, 128, False)["block_m"] == 128
    assert fa.plan(4, 12, 4096, 64, True, 64, 64, 4)["key_split"] == 2  # forced
    assert fa.plan(1, 1, 8, 64, True, 128, 64, 4)["key_split"] == 1


def test_plan_head_groups():
    # heads per XCD group: the largest divisor of B*H/8 whose K and V (T * d * 2 bytes each) fit in
    # 16 MB when causal, 2 MB otherwise; 1 when B*H is not a multiple of 8
    def hg(B, H, T, d, causal):
        return fa.plan(B, H, T, d, causal)["head_group"]
    MiB = 1 << 20

    def expect(B, H, T, d, causal):
        if B * H == 0 or (B * H) % 8:
            return 1
        per, kv = B * H // 8, T * d * 2 * 2
        gmax = max(1, (16 * MiB if causal else 2 * MiB) // kv)
        return max(g for g in range(1, per + 1) if per % g == 0 and (g <= gmax or g == 1))
    cases = [(4, 12, 4096, 64, True, 6),      # 1 MB per head: all 6 of the XCD's heads
             (4, 12, 8192, 64, True, 6),      # 2 MB
             (4, 12, 16384, 64, True, 3),     # 4 MB: at most 4 heads, a divisor of 6
             (4, 16, 32768, 64, True, 2),     # 8 MB
             (1, 32, 65536, 64, True, 1),     # 16 MB
             (4, 16, 8192, 128, True, 4),     # 4 MB at d = 128
             (4, 16, 16384, 128, True, 2),
             (4, 16, 8192, 128, False, 1),    # non-causal: 2 MB budget, 4 MB per head
             (4, 16, 2048, 64, False, 4),     # non-causal: 512 KB per head, 4 fit, a divisor of 8
             (3, 12, 4096, 64, True, 1),      # B*H = 36: not a multiple of 8
             (1, 8, 1000, 64, True, 1),       # one head per XCD
             (0, 8, 1000, 64, True, 1)]       # no heads: nothing is launched, the plan says 1
    for B, H, T, d, causal, want in cases:
        assert hg(B, H, T, d, causal) == want == expect(B, H, T, d, causal), (B, H, T, d, causal)
    rng = np.random.default_rng(8)  # and a seeded sweep of shapes against the rule as written above
    for _ in range(500):
        B, H = int(rng.integers(1, 9)), int(rng.integers(1, 65))
        T, d, causal = int(rng.integers(1, 1 << 17)), int(rng.choice([64, 128])), bool(rng.integers(0, 2))
        assert hg(B, H, T, d, causal) == expect(B, H, T, d, causal), (B, H, T, d, causal)


def test_plan_errors():
    with pytest.raises(fa.FaError) as e:
        fa.plan(1, 1, 8, 80)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED_D
    with pytest.raises(fa.FaError) as e:
        fa.plan(1, 1, 8, 64, True, 96, 64, 3)
    assert e.value.status == fa.FA_ERR_TILE
    assert fa.lib().fa_fwd_plan(1, 1, 8, 64, 1, 0, 0, 0, None) == fa.FA_ERR_NULL


# ---- fa_bwd: the same checks, before anything is launched
BW = dict(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, dout=6 * A, dq=7 * A, dk=8 * A, dv=9 * A,
          delta=10 * A)


def call_bwd(B=1, H=1, T=8, d=64, causal=1, scale=0.125, **kw):
    p = dict(BW, **kw)
    return fa.lib().fa_bwd(p["q"], p["k"], p["v"], p["o"], p["lse"], p["dout"], p["dq"], p["dk"],
                           p["dv"], p["delta"], B, H, T, d, causal, scale, None)


def test_bwd_null_pointers():
    for name in BW:
        assert call_bwd(**{name: None}) == fa.FA_ERR_NULL, name


def test_bwd_sizes_head_dim_scale():
    assert call_bwd(T=-1) == fa.FA_ERR_INVALID_ARG
    assert call_bwd(B=1 << 13, H=1 << 12) == fa.FA_ERR_INVALID_ARG
    assert call_bwd(d=96) == fa.FA_ERR_UNSUPPORTED_D  # the backward takes d = 64 or 128
    assert call_bwd(d=32) == fa.FA_ERR_UNSUPPORTED_D
    for sc in (0.0, -1.0, float("nan"), float("inf"), 3.0e38):
        assert call_bwd(scale=sc) == fa.FA_ERR_INVALID_ARG


def test_bwd_alignment():
    for name in ("q", "k", "v", "o", "dout", "dq", "dk", "dv"):
        assert call_bwd(**{name: BW[name] + 8}) == fa.FA_ERR_ALIGNMENT, name
    for name in ("lse", "delta"):
        assert call_bwd(**{name: BW[name] + 2}) == fa.FA_ERR_ALIGNMENT, name
        assert call_bwd(T=0, **{name: BW[name] + 4}) == fa.FA_OK, name


def test_bwd_overlaps():
    # each bf16 tensor is 1 KiB at T=8, d=64; lse/delta 32 B
    assert call_bwd(dq=A + 512) == fa.FA_ERR_INVALID_ARG       # output over an input
    assert call_bwd(dk=7 * A + 256) == fa.FA_ERR_INVALID_ARG   # output over another output
    assert call_bwd(delta=5 * A + 16) == fa.FA_ERR_INVALID_ARG  # over lse
    assert call_bwd(delta=9 * A + 1020) == fa.FA_ERR_INVALID_ARG  # over dv


@pytest.mark.parametrize("shape", [(0, 3, 8, 64), (2, 0, 8, 64), (2, 3, 0, 64)])
def test_bwd_empty_problem_is_ok(shape):
    B, H, T, d = shape
    assert call_bwd(B=B, H=H, T=T, d=d) == fa.FA_OK
    assert call_bwd(B=B, H=H, T=T, d=d, causal=0) == fa.FA_OK


# ---- fa_fwd_sparse: checks before anything is launched
def call_sparse(B=1, H=1, T=8, d=64, causal=1, scale=0.125, mask=6 * A, mask_heads=1, **kw):
    p = dict(dict(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A), **kw)
    return fa.lib().fa_fwd_sparse(p["q"], p["k"], p["v"], p["o"], p["lse"], B, H, T, d, causal, scale,
                                  mask, mask_heads, None)


def test_sparse_checks():
    assert call_sparse(mask=None) == fa.FA_ERR_NULL
    assert call_sparse(o=None) == fa.FA_ERR_NULL
    assert call_sparse(d=96) == fa.FA_ERR_UNSUPPORTED_D
    assert call_sparse(T=65537) == fa.FA_ERR_INVALID_ARG      # above FA_SPARSE_MAX_T
    assert call_sparse(mask_heads=2) == fa.FA_ERR_INVALID_ARG  # neither 1 nor B*H
    assert call_sparse(B=2, H=3, mask_heads=6, T=0) == fa.FA_OK
    assert call_sparse(scale=0.0) == fa.FA_ERR_INVALID_ARG
    assert call_sparse(scale=3.0e38) == fa.FA_ERR_INVALID_ARG
    assert call_sparse(q=A + 8) == fa.FA_ERR_ALIGNMENT
    assert call_sparse(o=6 * A) == fa.FA_ERR_INVALID_ARG      # output over the mask
    assert call_sparse(T=0) == fa.FA_OK and call_sparse(T=0, d=128, causal=0) == fa.FA_OK
    assert fa.sparse_mask_shape(1000, 1) == (1, 8, 16) and fa.sparse_mask_shape(64, 12) == (12, 1, 1)


# ---- fa_fwd_partial and fa_merge: checks before anything is launched
def call_partial(B=1, H=1, T=200, Tk=None, d=64, causal=1, scale=0.125, k_begin=0, k_end=200, **kw):
    p = dict(dict(q=A, k=2 * A, v=3 * A, o=8 * A, lse=12 * A), **kw)
    Tk = T if Tk is None else Tk
    return fa.lib().fa_fwd_partial(p["q"], p["k"], p["v"], p["o"], p["lse"], B, H, T, Tk, d, causal,
                                   scale, k_begin, k_end, None)


def test_partial_checks():
    assert call_partial(T=0, k_end=0) == fa.FA_OK
    assert call_partial(o=None) == fa.FA_ERR_NULL
    assert call_partial(k_begin=32) == fa.FA_ERR_INVALID_ARG      # not on a 64-key boundary
    assert call_partial(k_end=100) == fa.FA_ERR_INVALID_ARG       # neither aligned nor T
    assert call_partial(k_begin=128, k_end=64) == fa.FA_ERR_INVALID_ARG
    assert call_partial(k_end=256) == fa.FA_ERR_INVALID_ARG       # past T
    assert call_partial(k_begin=-64) == fa.FA_ERR_INVALID_ARG
    assert call_partial(d=32) == fa.FA_ERR_UNSUPPORTED_D
    assert call_partial(o=8 * A + 4) == fa.FA_ERR_ALIGNMENT
    assert call_partial(o=A) == fa.FA_ERR_INVALID_ARG             # fp32 output over q
    assert call_partial(T=4, Tk=-1, k_end=0) == fa.FA_ERR_INVALID_ARG
    assert call_partial(T=4, Tk=100, k_end=200) == fa.FA_ERR_INVALID_ARG  # range past Tk
    assert call_partial(T=0, Tk=100, k_end=100) == fa.FA_OK         # no query: nothing launched
    for sc in (0.0, float("inf"), 3.0e38):                          # 3e38 * log2(e) overflows fp32
        assert call_partial(scale=sc) == fa.FA_ERR_INVALID_ARG


def call_splitkv(B=1, H=2, T=4, Tk=1000, d=64, n=4, ws=16 * A, ws_bytes=None, **kw):
    p = dict(dict(q=A, k=2 * A, v=3 * A, o=8 * A, lse=12 * A), **kw)
    if ws_bytes is None:
        ws_bytes = fa.lib().fa_splitkv_workspace_bytes(B, H, T, d, max(n, 1))
    return fa.lib().fa_fwd_splitkv(p["q"], p["k"], p["v"], p["o"], p["lse"], B, H, T, Tk, d, 1, 0.125, n,
                                   ws, ws_bytes, None)


def test_splitkv_checks():
    lib = fa.lib()
    assert lib.fa_splitkv_workspace_bytes(2, 3, 5, 64, 4) == 4 * 2 * 3 * 5 * 65 * 4
    assert lib.fa_splitkv_workspace_bytes(2, 3, 5, 64, 0) == 0
    assert lib.fa_splitkv_workspace_bytes(-1, 3, 5, 64, 1) == 0
    # sizes fa_fwd_splitkv rejects give 0, never a wrapped product
    assert lib.fa_splitkv_workspace_bytes(2, 3, 5, 96, 1) == 0
    assert lib.fa_splitkv_workspace_bytes(2, 3, 5, 64, 4097) == 0
    assert lib.fa_splitkv_workspace_bytes(1, 1, (1 << 22) + 1, 64, 1) == 0
    assert lib.fa_splitkv_workspace_bytes(1 << 13, 1 << 12, 1, 64, 1) == 0
    assert lib.fa_splitkv_workspace_bytes(1 << 30, 1 << 30, 1 << 30, 64, 1) == 0
    # the largest accepted sizes: one part fits, 4096 of them (65 * 2^60 bytes) do not
    assert lib.fa_splitkv_workspace_bytes(1 << 12, 1 << 12, 1 << 22, 64, 1) == (1 << 46) * 65 * 4
    assert lib.fa_splitkv_workspace_bytes(1 << 12, 1 << 12, 1 << 22, 64, 4096) == 0
    assert call_splitkv(T=0) == fa.FA_OK
    assert call_splitkv(ws=None) == fa.FA_ERR_NULL
    assert call_splitkv(n=0) == fa.FA_ERR_INVALID_ARG
    assert call_splitkv(n=4097) == fa.FA_ERR_INVALID_ARG
    assert call_splitkv(ws_bytes=100) == fa.FA_ERR_INVALID_ARG     # workspace too small
    assert call_splitkv(d=96) == fa.FA_ERR_UNSUPPORTED_D
    assert call_splitkv(ws=16 * A + 8) == fa.FA_ERR_ALIGNMENT
    assert call_splitkv(o=8 * A + 2) == fa.FA_ERR_ALIGNMENT
    assert call_splitkv(o=16 * A) == fa.FA_ERR_INVALID_ARG         # output over the workspace
    assert call_splitkv(Tk=-5) == fa.FA_ERR_INVALID_ARG


def test_splitkv_split_count():
    lib = fa.lib()
    # few query blocks against many keys: split up to 512 workgroups, 512 keys per range at least
    assert lib.fa_splitkv_splits(1, 1, 1, 65536, 64) == 128
    assert lib.fa_splitkv_splits(1, 1, 1, 1 << 20, 64) == 256   # at most 256 ranges
    assert lib.fa_splitkv_splits(4, 12, 1, 65536, 64) == 10
    assert lib.fa_splitkv_splits(4, 12, 4096, 4096, 64) == 1
    assert lib.fa_splitkv_splits(1, 1, 1, 100, 64) == 1
    assert lib.fa_splitkv_splits(0, 1, 1, 100, 64) == 1
    # out-of-range sizes (no overflow in the tile counts)
    assert lib.fa_splitkv_splits(1, 1, 2 ** 31 - 1, 100, 64) == 1
    assert lib.fa_splitkv_splits(1, 1, 1, 2 ** 31 - 1, 64) == 1
    assert lib.fa_splitkv_splits(1, 1, 1, 65536, 96) == 1


def call_merge(n=2, B=1, H=1, T=8, d=64, **kw):
    p = dict(dict(op=A, lp=4 * A, o=6 * A, lse=8 * A), **kw)
    return fa.lib().fa_merge(p["op"], p["lp"], n, p["o"], p["lse"], B, H, T, d, None)


def test_merge_checks():
    assert call_merge(T=0) == fa.FA_OK
    assert call_merge(n=0) == fa.FA_ERR_INVALID_ARG
    assert call_merge(n=4097) == fa.FA_ERR_INVALID_ARG
    assert call_merge(op=None) == fa.FA_ERR_NULL
    assert call_merge(d=96) == fa.FA_ERR_UNSUPPORTED_D
    assert call_merge(o=6 * A + 8) == fa.FA_ERR_ALIGNMENT
    assert call_merge(lse=8 * A + 2) == fa.FA_ERR_ALIGNMENT
    assert call_merge(o=A + 1024) == fa.FA_ERR_INVALID_ARG       # over the partial outputs


def call_fp8(B=1, H=1, T=200, d=64, causal=1, scale=0.125, qd=0.01, kd=0.01, vd=0.01, **kw):
    p = dict(dict(q=A, k=2 * A, v=3 * A, o=8 * A, lse=12 * A), **kw)
    return fa.lib().fa_fwd_fp8(p["q"], p["k"], p["v"], p["o"], p["lse"], B, H, T, d, causal, scale,
                               qd, kd, vd, None)


def test_fp8_checks():
    assert call_fp8(T=0) == fa.FA_OK
    assert call_fp8(v=None) == fa.FA_ERR_NULL
    assert call_fp8(d=96) == fa.FA_ERR_UNSUPPORTED_D
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert call_fp8(qd=bad) == fa.FA_ERR_INVALID_ARG
        assert call_fp8(vd=bad) == fa.FA_ERR_INVALID_ARG
        assert call_fp8(scale=bad) == fa.FA_ERR_INVALID_ARG
    assert call_fp8(qd=1e-30, kd=1e-30) == fa.FA_ERR_INVALID_ARG   # score factor underflows fp32
    assert call_fp8(scale=1e38, qd=2.0, kd=2.0) == fa.FA_ERR_INVALID_ARG  # and overflows it
    assert call_fp8(scale=1e30, qd=1.0, kd=1.0, T=0) == fa.FA_OK    # within range: accepted
    assert call_fp8(k=2 * A + 8) == fa.FA_ERR_ALIGNMENT
    assert call_fp8(lse=12 * A + 2) == fa.FA_ERR_ALIGNMENT
    assert call_fp8(o=A + 64) == fa.FA_ERR_INVALID_ARG             # output over q


NOALLOC_SCRATCH_BYTES = 64 << 20  # include/fa.h: FA_NOALLOC_SCRATCH_BYTES


def call_noalloc(B=1, H=2, T=4, Tk=1000, d=64, n=4, scale=0.125, **kw):
    p = dict(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A)
    p.update(kw)
    return fa.lib().fa_fwd_splitkv_noalloc(p["q"], p["k"], p["v"], p["o"], p["lse"], B, H, T, Tk, d, 1,
                                           scale, n, None)


def test_splitkv_noalloc_checks():
    # every rejection happens before the scratch buffer is looked up (no HIP call on any of these)
    for kw in ("q", "k", "v", "o", "lse"):
        assert call_noalloc(**{kw: None}) == fa.FA_ERR_NULL
    assert call_noalloc(n=0) == fa.FA_ERR_INVALID_ARG
    assert call_noalloc(n=4097) == fa.FA_ERR_INVALID_ARG
    assert call_noalloc(T=-1) == fa.FA_ERR_INVALID_ARG
    assert call_noalloc(Tk=-1) == fa.FA_ERR_INVALID_ARG
    assert call_noalloc(Tk=(1 << 22) + 1) == fa.FA_ERR_INVALID_ARG
    assert call_noalloc(d=96) == fa.FA_ERR_UNSUPPORTED_D
    assert call_noalloc(scale=0.0) == fa.FA_ERR_INVALID_ARG
    assert call_noalloc(scale=float("nan")) == fa.FA_ERR_INVALID_ARG
    assert call_noalloc(scale=3.0e38) == fa.FA_ERR_INVALID_ARG
    assert call_noalloc(q=A + 8) == fa.FA_ERR_ALIGNMENT
    assert call_noalloc(lse=5 * A + 2) == fa.FA_ERR_ALIGNMENT
    # an empty problem is a no-op
    assert call_noalloc(T=0) == fa.FA_OK
    assert call_noalloc(B=0) == fa.FA_OK


def test_splitkv_noalloc_rejects_problems_beyond_its_scratch():
    lib = fa.lib()
    # the largest split count whose partial results fit, and one more
    B, H, T, d = 4, 16, 64, 128
    per_split = lib.fa_splitkv_workspace_bytes(B, H, T, d, 1)
    n_fit = NOALLOC_SCRATCH_BYTES // per_split
    assert lib.fa_splitkv_workspace_bytes(B, H, T, d, n_fit) <= NOALLOC_SCRATCH_BYTES
    assert lib.fa_splitkv_workspace_bytes(B, H, T, d, n_fit + 1) > NOALLOC_SCRATCH_BYTES
    assert call_noalloc(B=B, H=H, T=T, Tk=1 << 16, d=d, n=n_fit + 1) == fa.FA_ERR_SCRATCH
    assert call_noalloc(B=1, H=1, T=1 << 22, Tk=1 << 22, d=128, n=1) == fa.FA_ERR_SCRATCH
    assert "FA_NOALLOC_SCRATCH_BYTES" in fa.strerror(fa.FA_ERR_SCRATCH)

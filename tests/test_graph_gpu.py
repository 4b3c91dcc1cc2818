"""The entry points inside a captured HIP graph (torch.cuda.graph over the C-ABI calls).

The library launches kernels only: no allocation, no memset, no synchronisation, so a call can be
captured on the capture stream and replayed. Each test captures once with static buffers, then
replays several times; between replays the inputs are overwritten by eager copies and the program
synchronises, and every replay must equal an eager call on the same inputs bit for bit (every
launch here is deterministic).
"""
import pytest
import torch

import exact_tiled_attention_07_amd as fa
from exact_tiled_attention_07_amd.inputs import make_qkv, to_torch_bf16

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REPLAYS = 4


def capture(fn):
    """Warm fn up on a side stream, then capture it into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def assert_same(a, b, label):
    assert torch.equal(bits(a), bits(b)), label


def fill(dst_tensors, B, H, T, d, seed):
    for dst, src in zip(dst_tensors, make_qkv(B, H, T, d, seed=seed)):
        dst.copy_(to_torch_bf16(src, DEV))


@pytest.mark.parametrize("B,H,T,d,causal", [(2, 3, 1000, 64, True), (1, 2, 300, 128, False),
                                            (1, 2, 40, 64, True), (4, 12, 1024, 64, True)])
def test_fwd_graph_replays(B, H, T, d, causal):
    # the default launch of each shape: the key split, 128 x 64 (d = 128), 128 x 64, 128 x 128
    assert d == 128 or [fa.plan(B, H, T, d, causal)[x] for x in ("key_split", "block_n")] == {
        1000: [2, 64], 40: [1, 64], 1024: [1, 128]}[T]
    q, k, v = (torch.empty(B, H, T, d, dtype=torch.bfloat16, device=DEV) for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty(B, H, T, dtype=torch.float32, device=DEV)
    fill((q, k, v), B, H, T, d, seed=1)
    g = capture(lambda: fa.fwd(q, k, v, causal=causal, out=o, lse=lse))
    for r in range(REPLAYS):
        fill((q, k, v), B, H, T, d, seed=100 + r)
        o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        o_e, lse_e = fa.fwd(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert_same(o, o_e, f"o, replay {r}")
        assert_same(lse, lse_e, f"lse, replay {r}")


def test_splitkv_graph_replays():
    # two kernels (key ranges, then the merge) and a caller-owned workspace
    B, H, T, Tk, d = 2, 3, 4, 5000, 64
    q = torch.empty(B, H, T, d, dtype=torch.bfloat16, device=DEV)
    k, v = (torch.empty(B, H, Tk, d, dtype=torch.bfloat16, device=DEV) for _ in range(2))
    n = fa.splitkv_splits(B, H, T, Tk, d)
    assert n > 1
    ws = torch.empty(fa.splitkv_workspace_bytes(B, H, T, d, n), dtype=torch.uint8, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty(B, H, T, dtype=torch.float32, device=DEV)

    def refill(seed):
        qb, _, _ = make_qkv(B, H, T, d, seed=seed)
        _, kb, vb = make_qkv(B, H, Tk, d, seed=seed + 1)
        for dst, src in zip((q, k, v), (qb, kb, vb)):
            dst.copy_(to_torch_bf16(src, DEV))

    refill(2)
    g = capture(lambda: fa.fwd_splitkv(q, k, v, causal=True, n_splits=n, out=o, lse=lse, workspace=ws))
    for r in range(REPLAYS):
        refill(200 + 2 * r)
        o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        o_e, lse_e = fa.fwd_splitkv(q, k, v, causal=True, n_splits=n)
        torch.cuda.synchronize()
        assert_same(o, o_e, f"o, replay {r}")
        assert_same(lse, lse_e, f"lse, replay {r}")


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_graph_replays(d):
    # the forward and both backward kernels in one graph
    B, H, T = 1, 3, 700
    q, k, v, do = (torch.empty(B, H, T, d, dtype=torch.bfloat16, device=DEV) for _ in range(4))
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse, delta = (torch.empty(B, H, T, dtype=torch.float32, device=DEV) for _ in range(2))

    def step():
        fa.fwd(q, k, v, causal=True, out=o, lse=lse)
        fa.bwd(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv, delta=delta)

    fill((q, k, v), B, H, T, d, seed=3)
    fill((do,), B, H, T, d, seed=4)
    g = capture(step)
    for r in range(REPLAYS):
        fill((q, k, v), B, H, T, d, seed=300 + r)
        fill((do,), B, H, T, d, seed=400 + r)
        for t in (dq, dk, dv):
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        o_e, lse_e = fa.fwd(q, k, v, causal=True)
        got = fa.bwd(q, k, v, o_e, lse_e, do, causal=True)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv", "delta"), (dq, dk, dv, delta), got):
            assert_same(a, b, f"{name}, replay {r}")


def test_fp8_graph_replays():
    from exact_tiled_attention_07_amd.inputs import make_qkv_fp8
    B, H, T, d = 2, 2, 900, 64
    q, k, v = (torch.empty(B, H, T, d, dtype=torch.uint8, device=DEV) for _ in range(3))
    o = torch.empty(B, H, T, d, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, H, T, dtype=torch.float32, device=DEV)

    def refill(seed):
        q8, k8, v8, sc = make_qkv_fp8(B, H, T, d, seed=seed)
        for dst, src in zip((q, k, v), (q8, k8, v8)):
            dst.copy_(torch.from_numpy(src).to(DEV))
        return sc

    sc = refill(7)
    # the descale factors are launch arguments, fixed at capture: replays reuse the captured ones
    g = capture(lambda: fa.fwd_fp8(q, k, v, *sc, causal=True, out=o, lse=lse))
    for r in range(REPLAYS):
        refill(700 + r)
        o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        o_e, lse_e = fa.fwd_fp8(q, k, v, *sc, causal=True)
        torch.cuda.synchronize()
        assert_same(o, o_e, f"o, replay {r}")
        assert_same(lse, lse_e, f"lse, replay {r}")


def test_sparse_partial_merge_noalloc_graph_replays():
    # the remaining entry points in one graph: the block-sparse forward, two partials and their
    # merge (into static fp32 part buffers), and the no-alloc split-KV call
    from exact_tiled_attention_07_amd.inputs import sparse_mask

    B, H, T, d = 1, 3, 700, 64
    q, k, v = (torch.empty(B, H, T, d, dtype=torch.bfloat16, device=DEV) for _ in range(3))
    qn = torch.empty(B, H, 5, d, dtype=torch.bfloat16, device=DEV)
    mask = torch.from_numpy(sparse_mask(T, 0.4, 3)).to(DEV)
    o_s, o_m, o_n = (torch.empty(B, H, t, d, dtype=torch.bfloat16, device=DEV) for t in (T, T, 5))
    l_s, l_m, l_n = (torch.empty(B, H, t, dtype=torch.float32, device=DEV) for t in (T, T, 5))
    op = torch.empty(2, B, H, T, d, dtype=torch.float32, device=DEV)
    lp = torch.empty(2, B, H, T, dtype=torch.float32, device=DEV)

    def refill(seed):
        fill((q, k, v), B, H, T, d, seed)
        qn.copy_(to_torch_bf16(make_qkv(B, H, 5, d, seed=seed + 1)[0], DEV))

    def calls():
        fa.fwd_sparse(q, k, v, mask, causal=True, out=o_s, lse=l_s)
        for i, (a, b) in enumerate(((0, 320), (320, T))):
            fa.fwd_partial(q, k, v, a, b, causal=True, o_part=op[i], lse_part=lp[i])
        fa.merge(op, lp, out=o_m, lse=l_m)
        fa.fwd_splitkv_noalloc(qn, k, v, causal=True, n_splits=6, out=o_n, lse=l_n)

    refill(11)
    g = capture(calls)
    for r in range(REPLAYS):
        refill(1100 + r)
        for t in (o_s, o_m, o_n):
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        e_s = fa.fwd_sparse(q, k, v, mask, causal=True)
        parts = [fa.fwd_partial(q, k, v, a, b, causal=True) for a, b in ((0, 320), (320, T))]
        e_m = fa.merge(torch.stack([p[0] for p in parts]), torch.stack([p[1] for p in parts]))
        e_n = fa.fwd_splitkv(qn, k, v, causal=True, n_splits=6)
        torch.cuda.synchronize()
        for (got_o, got_l), (want_o, want_l), name in (((o_s, l_s), e_s, "sparse"), ((o_m, l_m), e_m, "merge"),
                                                         ((o_n, l_n), e_n, "noalloc splitkv")):
            assert_same(got_o, want_o, f"{name} o, replay {r}")
            assert_same(got_l, want_l, f"{name} lse, replay {r}")

"""Several host threads calling the library at once, each on its own stream (through the C-ABI).

The header states that the library keeps no mutable global state beyond the no-alloc buffer's
address and is safe to call from several host threads. Here four threads each run every entry point
that takes its buffers from the caller (forward, its forced-tile form, backward, block-sparse,
partial and merge, split-KV with its own workspace, FP8), on inputs of their own, several times
over, all at the same time; the ctypes calls release the GIL, so the argument checks and launches
interleave for real. Every kernel is deterministic, so each result must equal, bit for bit, that of
the same calls made one thread at a time beforehand.
"""
import threading

import pytest
import torch

import exact_tiled_attention_07_amd as fa
from exact_tiled_attention_07_amd.inputs import make_qkv, make_qkv_fp8, sparse_mask, to_torch_bf16

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
THREADS, REPEATS = 4, 5


def make_job(t):
    """The inputs of thread t and a function running every entry point on a given stream."""
    B, H, T, d = 1 + t % 2, 3, 700 + 97 * t, 64 if t % 2 == 0 else 128
    qb, kb, vb = make_qkv(B, H, T, d, seed=300 + t)
    dob, _, _ = make_qkv(B, H, T, d, seed=400 + t)
    q, k, v, do = (to_torch_bf16(x, DEV) for x in (qb, kb, vb, dob))
    qn = to_torch_bf16(make_qkv(B, H, 3, d, seed=500 + t)[0], DEV)  # a few queries over the T keys
    mask = torch.from_numpy(sparse_mask(T, 0.4, 600 + t)).to(DEV)
    q8, k8, v8, sc = make_qkv_fp8(B, H, T, d, seed=700 + t)
    q8, k8, v8 = (torch.from_numpy(x).to(DEV) for x in (q8, k8, v8))
    ws = torch.empty(fa.splitkv_workspace_bytes(B, H, 3, d, 4), dtype=torch.uint8, device=DEV)

    def run(stream):
        with torch.cuda.stream(stream):
            o, lse = fa.fwd(q, k, v, causal=True, stream=stream)
            o2, _ = fa.fwd_ex(q, k, v, 128, 64, 4, causal=False, stream=stream)
            dq, dk, dv, _ = fa.bwd(q, k, v, o, lse, do, causal=True, stream=stream)
            os_, _ = fa.fwd_sparse(q, k, v, mask, causal=True, stream=stream)
            parts = [fa.fwd_partial(q, k, v, a, b, causal=True, stream=stream)
                     for a, b in ((0, 256), (256, T))]
            om, _ = fa.merge(torch.stack([p[0] for p in parts]), torch.stack([p[1] for p in parts]),
                             stream=stream)
            od, _ = fa.fwd_splitkv(qn, k, v, causal=True, n_splits=4, workspace=ws, stream=stream)
            o8, _ = fa.fwd_fp8(q8, k8, v8, *sc, causal=True, stream=stream)
        return [o, lse, o2, dq, dk, dv, os_, om, od, o8]

    return run


def test_concurrent_host_threads():
    jobs = [make_job(t) for t in range(THREADS)]
    torch.cuda.synchronize()  # the inputs are in place before other streams read them
    # one thread at a time first: the reference results
    ref = []
    for job in jobs:
        s = torch.cuda.Stream()
        ref.append(job(s))
        s.synchronize()
    results = [[None] * REPEATS for _ in range(THREADS)]
    errors = []
    start = threading.Barrier(THREADS)

    def worker(t):
        try:
            s = torch.cuda.Stream()
            start.wait()
            for r in range(REPEATS):
                results[t][r] = jobs[t](s)
            s.synchronize()
        except Exception as e:  # reported below, after every thread has ended
            errors.append((t, repr(e)))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    names = ["fwd o", "fwd lse", "fwd_ex o", "bwd dq", "bwd dk", "bwd dv", "sparse o", "merge o",
             "splitkv o", "fp8 o"]
    for t in range(THREADS):
        for r in range(REPEATS):
            for name, got, want in zip(names, results[t][r], ref[t]):
                assert torch.equal(got, want), (t, r, name)
    print(f"[gpu threads] {THREADS} threads x {REPEATS} rounds x {len(names)} outputs: all equal to "
          "the one-thread results", flush=True)

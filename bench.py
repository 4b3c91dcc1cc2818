"""Benchmark of the exact attention forward on one MI355X.

A step is one fa_fwd call over the whole workload (all heads), inputs already resident in HBM.
Warm-up runs the given number of steps and then more until 0.3 s have passed (the shader clock rises
over the first part of a load); exactly `--steps` steps are timed. Prints one JSON line:
  value        counted TFLOP/s of the step (2*B*H*T^2*d causal, 4*B*H*T^2*d non-causal)
  roofline     the kernel's achieved TFLOP/s from one pair of HIP events on its launch stream
               around the timed launches, against the dense bf16 MFMA peak; traffic = HBM bytes
               per launch from rocprofv3 counters (when they were taken on the current kernel
               sources), else null; the same holds for clock_mhz, the shader clock measured under
               the kernel, and the fraction of the MFMA peak at that clock
  cpu_baseline the CPU oracle timed on the host cores on a bounded sample of the same workload
               (per_config: the oracle on every workload, and on one thread for the smallest)
  parity       the timed launch's output against that same oracle output, every row of the
               sampled heads (all of them at T=4096): literal max errors, the number of elements
               admitted only by the one-ulp clause, and the number of failures
  sweep        the same measurement at the other sequence lengths of the metric (T = 1024, 2048,
               8192, 16384) and on the d=128 workload (non-causal, and its causal variant)
  backward     fa_bwd (dQ, dK, dV from the forward's O and LSE) on the same workload: counted
               TFLOP/s with the usual 2.5x-forward count, per-launch HIP events around both kernels;
               d128: the same on the non-causal d=128 workload
  sparse       fa_fwd_sparse at T=16384 (B4 H12 d64 causal) under a seeded block mask (25% of the
               128x64 blocks plus the diagonal ones): TFLOP/s over the visible (query, key) pairs
               and the time against the dense forward of the same shape
  splitkv      fa_fwd_splitkv on decode shapes (1 and 16 queries after 16384 keys) against the HBM
               roofline, and the T=16384 workload as 4 key shards plus fa_merge
  fp8          fa_fwd_fp8 on E4M3 copies of the T=4096, 16384 and d=128 workloads against the FP8
               MFMA peak, with fa_fwd on the bf16 inputs timed alongside
  context      the source pages' own hardware claims (other GPUs), quoted as context only

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4] [--no-cpu-baseline]
                       [--no-sweep] [--no-backward] [--only-backward] [--no-sparse] [--no-splitkv]
                       [--no-fp8]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PEAK_FP8_TFLOPS = 5033.2   # MI355X dense fp8 MFMA: twice the bf16 rate
# What the source pages claim about their own hardware: quoted in the line as context only (other
# GPUs, no number for this metric); none of it is a target.
PAGE_CLAIMS = [
    {"claim": "best tile 128 query rows x 64 keys (B_r x B_c)", "hardware": "A100",
     "source": "ijyty.com FlashAttention article, section 1",
     "here": "the default tile on MI355X is also 128 x 64 (chosen by occupancy and measurement)"},
    {"claim": "more than 30% slower when B_r exceeds 256 (register spills)", "hardware": "A100",
     "source": "ijyty.com FlashAttention article, section 1"},
    {"claim": "memory bandwidth utilisation from 65% to 89% after 128-byte aligned loads, bank-conflict "
              "avoidance and asynchronous prefetch", "hardware": "A100",
     "source": "ijyty.com FlashAttention article, section 3.2"},
    {"claim": "3072 programs per launch at B4 H12 T4096 with 64 x 64 tiles", "hardware": "any",
     "source": "learn-llm.fim.ai, STEP 3"},
    {"claim": "the hand-written Triton kernel runs about as fast as PyTorch SDPA (FlashAttention-2)",
     "hardware": "RTX 4090", "source": "learn-llm.fim.ai, STEP 5"},
]
# What identifies the profiled kernel: its source and its launch plan on the profiled workload
# (the host code around it may change without touching the kernel the counters were taken on).
KERNEL_SOURCES = ["exact_tiled_attention_07_amd/csrc/fa_kernel.hpp"]
BWD_FLOPS_PER_FWD = 2.5  # the usual count: the backward's matrix products are 2.5x the forward's
BWD_SOURCES = ["exact_tiled_attention_07_amd/csrc/fa_bwd_kernel.hpp"] + KERNEL_SOURCES
PROFILED_WORKLOAD = "c4"  # the workload of the committed counter summaries
BWD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_bwd_c4_hbm_traffic.txt")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_fwd_c4_hbm_traffic.txt")
FP8_SOURCES = ["exact_tiled_attention_07_amd/csrc/fa_fp8_kernel.hpp"] + KERNEL_SOURCES
FP8_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_fwd_fp8_c4_hbm_traffic.txt")
SPLITKV_SOURCES = KERNEL_SOURCES + ["exact_tiled_attention_07_amd/csrc/fa_merge_kernel.hpp"]
SPLITKV_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_fwd_splitkv_hbm_traffic.txt")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "fa_fwd_c4_sq_counters.txt")
MFMA_FLOP_PER_CLK = 256 * 4 * 1024  # dense bf16: 1024 flop per clock on each of the 1024 SIMDs


def profiled_plan():
    """Launch plan of the forward on the profiled workload (host logic of libfa, no GPU needed)."""
    import exact_tiled_attention_07_amd as fa
    from exact_tiled_attention_07_amd.inputs import WORKLOADS

    w = WORKLOADS[PROFILED_WORKLOAD]
    return fa.plan(w.B, w.H, w.T, w.d, w.causal)


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for rel in (KERNEL_SOURCES if sources is None else sources):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    h.update(json.dumps(profiled_plan(), sort_keys=True).encode())
    return h.hexdigest()[:16]


def recorded_traffic(path=None, sources=None, key="hbm_bytes_per_launch"):
    """HBM bytes per launch (or per call, under another key) from a committed counter summary, if
    taken on these sources."""
    path = TRAFFIC_FILE if path is None else path
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_hash:\s*(\w+)", text)
    m_bytes = re.search(re.escape(key) + r":\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash(sources):
        return None
    return float(m_bytes.group(1))


def recorded_clock_mhz():
    """Shader clock measured under this kernel (GRBM_GUI_ACTIVE per XCD over the traced duration),
    from the committed counter summary, if taken on these sources."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    text = open(COUNTERS_FILE).read()
    m_hash = re.search(r"kernel_source_hash:\s*(\w+)", text)
    m_clk = re.search(r"effective clock\s+([0-9.]+)\s*MHz", text)
    if not m_hash or not m_clk or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_clk.group(1))


MIN_WARM_S = 0.3  # warm-up spans at least this much wall time: the shader clock rises under load


def warm_up(step, warmup, sync, min_s=MIN_WARM_S):
    """Run `warmup` steps, then more in batches until at least `min_s` seconds have passed."""
    t0 = time.perf_counter()
    for _ in range(warmup):
        step()
    sync()
    n = max(1, warmup)
    while time.perf_counter() - t0 < min_s:
        for _ in range(n):
            step()
        sync()
        n = min(2 * n, 4096)


def time_region(step, steps, stream, sync):
    """Time exactly `steps` back-to-back launches: wall clock between two synchronisations, and one
    pair of HIP events on the launch stream around the same launches. Returns (wall ms per step,
    event ms per step); the event figure cannot exceed the wall figure by more than the events'
    own resolution, as nothing but the launches sits between them."""
    import torch

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sync()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    sync()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    return wall_ms, e0.elapsed_time(e1) / steps


def time_workload(wl, steps, warmup, tiles=None):
    """Returns (ms_per_step wall, kernel ms per launch from one event pair around the same timed
    launches, extra stats, (o, lse) of the last launch on the device)."""
    import torch

    import exact_tiled_attention_07_amd as fa
    from exact_tiled_attention_07_amd.inputs import to_torch_bf16

    dev = torch.device("cuda:0")
    qb, kb, vb = wl.make()
    q, k, v = (to_torch_bf16(x, dev) for x in (qb, kb, vb))
    del qb, kb, vb
    o = torch.empty_like(q)
    lse = torch.empty((wl.B, wl.H, wl.T), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)  # fa_fwd launches on this stream

    def step():
        if tiles is None:
            fa.fwd(q, k, v, causal=wl.causal, scale=wl.scale, out=o, lse=lse, stream=stream)
        else:
            fa.fwd_ex(q, k, v, *tiles, causal=wl.causal, scale=wl.scale, out=o, lse=lse, stream=stream)

    def sync():
        torch.cuda.synchronize(dev)

    warm_up(step, warmup, sync)
    wall_ms, kern_ms = time_region(step, steps, stream, sync)

    # per-launch event pairs (informational: the brackets themselves add a little time per launch)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    sync()
    durs = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))

    # one cold launch: flush L2/MALL by writing 512 MiB first
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    scratch.fill_(1)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    step()
    c1.record(stream)
    sync()
    cold_ms = c0.elapsed_time(c1)
    del scratch, q, k, v
    return wall_ms, kern_ms, {"per_launch_events": {"median_ms": round(durs[len(durs) // 2], 5),
                                                    "min_ms": round(durs[0], 5),
                                                    "max_ms": round(durs[-1], 5)},
                              "cold_ms": round(cold_ms, 5)}, (o, lse)


def time_backward(wl, steps, warmup):
    """fa_bwd on the workload's inputs (o and lse from one fa_fwd, dO drawn like the inputs).

    Returns (ms per fa_bwd call from one event pair on the launch stream around the timed calls,
    extra stats)."""
    import torch

    import exact_tiled_attention_07_amd as fa
    from exact_tiled_attention_07_amd.inputs import make_qkv, to_torch_bf16

    dev = torch.device("cuda:0")
    q, k, v = (to_torch_bf16(x, dev) for x in wl.make())
    do = to_torch_bf16(make_qkv(wl.B, wl.H, wl.T, wl.d, seed=wl.seed + 7919)[0], dev)
    o, lse = fa.fwd(q, k, v, causal=wl.causal, scale=wl.scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    delta = torch.empty_like(lse)
    stream = torch.cuda.current_stream(dev)

    def step():
        fa.bwd(q, k, v, o, lse, do, causal=wl.causal, scale=wl.scale, dq=dq, dk=dk, dv=dv,
               delta=delta, stream=stream)

    def sync():
        torch.cuda.synchronize(dev)

    warm_up(step, warmup, sync)
    wall_ms, ev_ms = time_region(step, steps, stream, sync)
    return ev_ms, {"wall_ms": wall_ms}


def visible_pairs(mask, T, causal):
    """Number of (query, key) pairs a block mask leaves visible (per head)."""
    import numpy as np

    nq, nk = mask.shape[1:]
    rows = np.arange(T)
    total = 0
    for qb in range(nq):
        r = rows[qb * 128:min(T, qb * 128 + 128)]
        for kb in np.nonzero(mask[0, qb])[0]:
            j0, j1 = kb * 64, min(T, kb * 64 + 64)
            if causal:
                total += int(np.clip(np.minimum(r + 1, j1) - j0, 0, None).sum())
            else:
                total += r.size * (j1 - j0)
    return total


def time_sparse(wl, steps, warmup, density=0.25):
    """fa_fwd_sparse vs fa_fwd on the same inputs; returns the bench line's `sparse` object."""
    import torch

    import exact_tiled_attention_07_amd as fa
    from exact_tiled_attention_07_amd.inputs import sparse_mask, to_torch_bf16

    dev = torch.device("cuda:0")
    q, k, v = (to_torch_bf16(x, dev) for x in wl.make())
    mask_np = sparse_mask(wl.T, density, wl.seed)
    mask = torch.from_numpy(mask_np).to(dev)
    o, lse = torch.empty_like(q), torch.empty((wl.B, wl.H, wl.T), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    timed = _event_timer(stream, steps, warmup)

    ms_sparse = timed(lambda: fa.fwd_sparse(q, k, v, mask, causal=wl.causal, scale=wl.scale, out=o,
                                            lse=lse, stream=stream))
    ms_dense = timed(lambda: fa.fwd(q, k, v, causal=wl.causal, scale=wl.scale, out=o, lse=lse,
                                    stream=stream))
    pairs = visible_pairs(mask_np, wl.T, wl.causal)
    flops = 4.0 * wl.d * pairs * wl.B * wl.H
    dense_pairs = wl.T * (wl.T + 1) // 2 if wl.causal else wl.T * wl.T
    return {"workload": wl.name, "mask": f"{density:.0%} random 128x64 blocks + diagonal, seed {wl.seed}",
            "visible_fraction": round(pairs / dense_pairs, 4), "ms_per_step": round(ms_sparse, 5),
            "tflops": round(flops / (ms_sparse * 1e-3) / 1e12, 3),
            "pct_of_peak": round(100 * flops / (ms_sparse * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "dense_ms": round(ms_dense, 5), "speedup_vs_dense": round(ms_dense / ms_sparse, 3)}


def _event_timer(stream, steps, warmup):
    """A timer for one entry point: time-based warm-up, then ms per call from one event pair around
    `steps` back-to-back calls on the launch stream."""
    import torch

    def sync():
        torch.cuda.synchronize(stream.device)

    def timed(fn):
        warm_up(fn, warmup, sync, min_s=0.1)
        return time_region(fn, steps, stream, sync)[1]
    return timed


def _graph_timer(steps, warmup):
    """A timer for calls too short to outrun their Python launch overhead: `steps` calls captured
    once into a HIP graph (each call launches on the current stream, the capture stream while
    capturing), then ms per call from one event pair around a replay of the graph."""
    import torch

    def timed(fn):
        fn()  # once eagerly, outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                fn()
        stream = torch.cuda.current_stream()
        warm_up(g.replay, max(1, warmup // max(steps, 1)), torch.cuda.synchronize, min_s=0.1)
        ms = time_region(g.replay, 1, stream, torch.cuda.synchronize)[1] / steps
        del g
        return ms
    return timed


# Decode-shaped split-KV workloads: a few new queries per sequence at the end of the 16384-key
# sequences of the B=4, H=12, d=64 workload (causal, the queries after the keys' prefix).
DECODE_SHAPES = ((4, 12, 1, 16384, 64), (4, 12, 16, 16384, 64))


def time_splitkv(steps, warmup):
    """fa_fwd_splitkv on decode shapes (vs one range, i.e. no split), and the T=16384 workload cut
    into 4 key shards (fa_fwd_partial x4 + fa_merge) vs fa_fwd. Returns the bench line's object."""
    import torch

    import exact_tiled_attention_07_amd as fa
    from exact_tiled_attention_07_amd.inputs import WORKLOADS, make_qkv, to_torch_bf16

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    gtimed = _graph_timer(max(steps, 50), warmup)
    decode = []
    for (B, H, T, Tk, d) in DECODE_SHAPES:
        q = to_torch_bf16(make_qkv(B, H, T, d, seed=91)[0], dev)
        _, kb, vb = make_qkv(B, H, Tk, d, seed=92)
        k, v = to_torch_bf16(kb, dev), to_torch_bf16(vb, dev)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
        n = fa.splitkv_splits(B, H, T, Tk, d)
        ws = torch.empty(fa.splitkv_workspace_bytes(B, H, T, d, n), dtype=torch.uint8, device=dev)
        # one call is a few tens of microseconds: timed as a graph of `steps` calls (no host gaps)
        ms = gtimed(lambda: fa.fwd_splitkv(q, k, v, causal=True, n_splits=n, out=o, lse=lse, workspace=ws))
        ms1 = gtimed(lambda: fa.fwd_splitkv(q, k, v, causal=True, n_splits=1, out=o, lse=lse, workspace=ws))
        # algorithmic HBM bytes: q, k, v read once, o and lse written once (the partial results'
        # round trip through the workspace is the split's own cost, so it is not counted)
        alg = B * H * (2 * T * d * 2 + 2 * Tk * d * 2 + T * 4)
        gbs = alg / (ms * 1e-3) / 1e9
        shape = f"B{B} H{H} T{T} Tk{Tk} d{d} causal"
        decode.append({"shape": shape, "n_splits": n,
                       "ms_per_step": round(ms, 5), "no_split_ms": round(ms1, 5),
                       "speedup_vs_no_split": round(ms1 / ms, 3),
                       "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                                    "traffic": recorded_traffic(SPLITKV_TRAFFIC_FILE, SPLITKV_SOURCES,
                                                                f"hbm_bytes_per_call[{shape}]"),
                                    "algorithmic_bytes": alg}})
        del ws
    wl = WORKLOADS["c5a"]
    q, k, v = (to_torch_bf16(x, dev) for x in wl.make())
    o, lse = torch.empty_like(q), torch.empty((wl.B, wl.H, wl.T), dtype=torch.float32, device=dev)
    shards = 4
    edges = [wl.T * i // shards for i in range(shards + 1)]
    op = torch.empty((shards, wl.B, wl.H, wl.T, wl.d), dtype=torch.float32, device=dev)
    lp = torch.empty((shards, wl.B, wl.H, wl.T), dtype=torch.float32, device=dev)

    def sharded():
        for i in range(shards):
            fa.fwd_partial(q, k, v, edges[i], edges[i + 1], causal=True, scale=wl.scale, o_part=op[i],
                           lse_part=lp[i], stream=stream)
        fa.merge(op, lp, out=o, lse=lse, stream=stream)

    few = max(3, steps // 10), max(2, warmup // 10)
    timed_few = _event_timer(stream, *few)
    ms_sh = timed_few(sharded)
    ms_merge = timed_few(lambda: fa.merge(op, lp, out=o, lse=lse, stream=stream))
    ms_dense = timed_few(lambda: fa.fwd(q, k, v, causal=True, scale=wl.scale, out=o, lse=lse, stream=stream))
    rows = wl.B * wl.H * wl.T
    merge_bytes = shards * rows * (wl.d + 1) * 4 + rows * (wl.d * 2 + 4)
    mgbs = merge_bytes / (ms_merge * 1e-3) / 1e9
    del op, lp
    return {"decode": decode,
            "key_shards": {"workload": wl.name, "shards": shards, "ms_per_step": round(ms_sh, 5),
                           "tflops": round(wl.flops / (ms_sh * 1e-3) / 1e12, 2), "dense_ms": round(ms_dense, 5),
                           "overhead_vs_dense": round(ms_sh / ms_dense, 3), "merge_ms": round(ms_merge, 5),
                           "merge_roofline": {"bound": "hbm", "achieved": round(mgbs, 1), "peak": PEAK_HBM_GBS,
                                              "unit": "GB/s", "frac": round(mgbs / PEAK_HBM_GBS, 4),
                                              "traffic": recorded_traffic(
                                                  SPLITKV_TRAFFIC_FILE, SPLITKV_SOURCES,
                                                  f"hbm_bytes_per_merge[{wl.name} x{shards}]"),
                                              "algorithmic_bytes": merge_bytes}}}


def time_fp8(names, steps, warmup):
    """fa_fwd_fp8 on FP8 copies of the workloads (same seeds, per-tensor E4M3 quantization), against
    the fp8 MFMA peak, with fa_fwd on the bf16 inputs of the same workload timed alongside."""
    import torch

    import exact_tiled_attention_07_amd as fa
    from exact_tiled_attention_07_amd.inputs import WORKLOADS, make_qkv_fp8, to_torch_bf16

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    out = {}
    for name in names:
        wl = WORKLOADS[name]
        few = (max(5, steps // 5), max(2, warmup // 5)) if wl.T > 4096 else (steps, warmup)
        timed = _event_timer(stream, *few)
        q8, k8, v8, sc = make_qkv_fp8(wl.B, wl.H, wl.T, wl.d, wl.seed, wl.sigma)
        t8 = [torch.from_numpy(x).to(dev) for x in (q8, k8, v8)]
        o = torch.empty((wl.B, wl.H, wl.T, wl.d), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((wl.B, wl.H, wl.T), dtype=torch.float32, device=dev)
        ms = timed(lambda: fa.fwd_fp8(*t8, *sc, causal=wl.causal, scale=wl.scale, out=o, lse=lse, stream=stream))
        q, k, v = (to_torch_bf16(x, dev) for x in wl.make())
        ms16 = timed(lambda: fa.fwd(q, k, v, causal=wl.causal, scale=wl.scale, out=o, lse=lse, stream=stream))
        tf = wl.flops / (ms * 1e-3) / 1e12
        out[name] = {"workload": wl.name + " (E4M3 inputs)", "ms_per_step": round(ms, 5), "tflops": round(tf, 2),
                     "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS,
                                  "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                                  "traffic": recorded_traffic(FP8_TRAFFIC_FILE, FP8_SOURCES) if name == PROFILED_WORKLOAD
                                  else None},
                     "bf16_ms": round(ms16, 5), "speedup_vs_bf16": round(ms16 / ms, 3)}
        del t8, q, k, v
    return out


def _oracle_flops(wl, T, rows_per_head, heads):
    """Counted flops (the metric's count) of `heads` heads, `rows_per_head` rows each."""
    import numpy as np

    i = np.arange(rows_per_head, dtype=np.float64)
    per_head = (4.0 * wl.d * (i + 1)).sum() if wl.causal else 4.0 * wl.d * T * rows_per_head
    return float(per_head * heads)


def cpu_baseline(wl, budget_s=20.0):
    """Time the CPU oracle on a bounded sample of the workload (whole heads, all host cores).

    Returns (the bench line's cpu_baseline object, oracle (o, lse) of the sampled heads, the number
    of sampled heads): the same oracle output is the reference of the bench's parity check."""
    import oracle

    threads = len(os.sched_getaffinity(0))
    qb, kb, vb = wl.make()
    d, T = wl.d, wl.T

    # probe with one head, then take as many whole heads as fit the time budget
    t0 = time.perf_counter()
    oracle.attention_fwd(qb[:1, :1], kb[:1, :1], vb[:1, :1], wl.causal, wl.scale, num_threads=threads)
    probe_s = time.perf_counter() - t0
    n_heads_total = wl.B * wl.H
    n_heads = max(1, min(n_heads_total, int(budget_s / max(probe_s, 1e-6))))
    flat = [x.reshape(1, n_heads_total, T, d)[:, :n_heads] for x in (qb, kb, vb)]
    t0 = time.perf_counter()
    o_ref, lse_ref = oracle.attention_fwd(*flat, wl.causal, wl.scale, num_threads=threads)
    dt = time.perf_counter() - t0
    fl = _oracle_flops(wl, T, T, n_heads)
    base = {"value": float(fl / dt / 1e12), "unit": "TFLOP/s", "cores": oracle.threads_used(threads),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{n_heads} of {n_heads_total} heads of {wl.name} (all {T} rows each), "
                      f"fp64 two-pass oracle, {dt:.1f} s"}
    return base, (o_ref, lse_ref), n_heads


PER_CONFIG = ("c1", "c2", "c3", "c4", "c5a", "c5b")


def compulsory_bytes(wl):
    """HBM bytes a launch cannot avoid: q, k, v read once, o and lse written once."""
    return wl.B * wl.H * (4 * wl.T * wl.d * 2 + 4 * wl.T)


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or the platform's processor string."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline_per_config(names=PER_CONFIG, budget_heads_s=3.0):
    """The oracle timed on every workload: C1-C4 whole (C1 also on one thread); C5a and C5b on whole
    heads of their shape (seeded N(0,1) draws of those heads), as many as fit about `budget_heads_s`
    seconds. The oracle's time does not depend on the values."""
    import oracle
    from exact_tiled_attention_07_amd.inputs import WORKLOADS, make_qkv

    threads = len(os.sched_getaffinity(0))
    out = {}
    for name in names:
        wl = WORKLOADS[name]
        for nt in ((threads, 1) if name == "c1" else (threads,)):
            if name in ("c5a", "c5b"):
                q1, k1, v1 = make_qkv(1, 1, wl.T, wl.d, seed=wl.seed + 1000)
                t0 = time.perf_counter()
                oracle.attention_fwd(q1, k1, v1, wl.causal, wl.scale, num_threads=nt)
                probe = time.perf_counter() - t0
                heads = max(1, min(wl.B * wl.H, int(budget_heads_s / max(probe, 1e-6))))
                qb, kb, vb = make_qkv(1, heads, wl.T, wl.d, seed=wl.seed + 1000)
                sample = f"{heads} of {wl.B * wl.H} heads of the {wl.name} shape (all rows)"
            else:
                qb, kb, vb = wl.make()
                heads = wl.B * wl.H
                sample = f"all of {wl.name}"
            t0 = time.perf_counter()
            oracle.attention_fwd(qb, kb, vb, wl.causal, wl.scale, num_threads=nt)
            dt = time.perf_counter() - t0
            fl = _oracle_flops(wl, wl.T, wl.T, heads)
            key = name if nt == threads else f"{name}_1thread"
            out[key] = {"value": round(fl / dt / 1e12, 5), "unit": "TFLOP/s",
                        "cores": oracle.threads_used(nt), "kind": "oracle", "seconds": round(dt, 3),
                        "sample": sample}
    return out


def parity_check(wl, o, lse, ref, n_heads):
    """The timed launch's output against the oracle output of the cpu_baseline leg (same inputs),
    over the heads the oracle computed, every row; the pages' tolerance (oracle/parity.py)."""
    from oracle.parity import compare, passed

    o_ref, lse_ref = ref
    BH = wl.B * wl.H
    og = o.reshape(BH, wl.T, wl.d)[:n_heads].float().cpu().numpy().reshape(o_ref.shape)
    lg = lse.reshape(BH, wl.T)[:n_heads].cpu().numpy().reshape(lse_ref.shape)
    st = compare(og, lg, o_ref, lse_ref)
    return {"workload": wl.name, "heads": n_heads, "rows": n_heads * wl.T, "elements": st["n"],
            "max_err_o": st["max_err_o"], "max_err_lse": st["max_err_lse"],
            "n_ulp_clause": st["n_ulp_clause"], "n_fail": st["n_fail_o"] + st["n_fail_lse"] + st["n_nonfinite"],
            "pass": passed(st),
            "tolerance": "|dO| <= 1.5e-2, or one bf16 ulp where |O_ref| >= 2; |dLSE| <= 1e-3",
            # relative RMS error of O: two bf16 roundings (P, then O) give at most 2^-7 / sqrt(12)
            # = 2.26e-3 for i.i.d. zero-mean V; the tests allow twice that
            "rms_rel_err_o": st["rms_err_o"] / st["rms_ref_o"] if st["rms_ref_o"] > 0 else 0.0}


def copy_calibration(mib):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    if not mib:
        return
    import torch

    src = torch.ones(mib << 20, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[bench] copy calibration: 3 copies of {mib} MiB", file=sys.stderr)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="c4")
    ap.add_argument("--tiles", default=None, help="force BMxBNxWAVES (fa_fwd_ex)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-sparse", action="store_true")
    ap.add_argument("--no-splitkv", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--only-backward", action="store_true",
                    help="time fa_bwd only and print its line (for profiling the backward)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this size (for counter calibration)")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the attention heads shard across GPUs with no exchange, so one GPU's share is the "
              "measured unit", file=sys.stderr)
        return 2

    import torch

    from exact_tiled_attention_07_amd.inputs import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    tiles = tuple(int(x) for x in args.tiles.split("x")) if args.tiles else None
    wl = WORKLOADS[args.workload]
    backward = None
    if not args.no_backward and wl.d == 64:
        bms, bex = time_backward(wl, args.steps, args.warmup)
        bfl = BWD_FLOPS_PER_FWD * wl.flops
        bach = bfl / (bms * 1e-3) / 1e12
        backward = {"workload": wl.name, "ms_per_step": round(bms, 5), "tflops": round(bach, 3),
                    "pct_of_peak": round(100 * bach / PEAK_BF16_TFLOPS, 2), "flops_counted": bfl,
                    **{k2: round(v2, 5) for k2, v2 in bex.items()},
                    "roofline": {"bound": "mfma", "achieved": round(bach, 3), "peak": PEAK_BF16_TFLOPS,
                                 "unit": "TFLOP/s", "frac": round(bach / PEAK_BF16_TFLOPS, 4),
                                 "traffic": recorded_traffic(BWD_TRAFFIC_FILE, BWD_SOURCES)
                                 if args.workload == PROFILED_WORKLOAD else None},
                    "kernel_source_hash": kernel_source_hash(BWD_SOURCES)}
        # the d = 128 backward on the non-causal d = 128 workload (fewer steps: ~5.5 TFLOP per call)
        w128 = WORKLOADS["c5b"]
        ms128, ex128 = time_backward(w128, max(5, args.steps // 20), max(2, args.warmup // 20))
        tf128 = BWD_FLOPS_PER_FWD * w128.flops / (ms128 * 1e-3) / 1e12
        backward["d128"] = {"workload": w128.name, "ms_per_step": round(ms128, 5), "tflops": round(tf128, 3),
                            "wall_ms": round(ex128["wall_ms"], 5),
                            "roofline": {"bound": "mfma", "achieved": round(tf128, 3), "peak": PEAK_BF16_TFLOPS,
                                         "unit": "TFLOP/s", "frac": round(tf128 / PEAK_BF16_TFLOPS, 4),
                                         "traffic": None}}
        print(f"[bench] backward {wl.name}: {backward}", file=sys.stderr, flush=True)
        if args.only_backward:
            copy_calibration(args.copy_calibration_mib)
            print(json.dumps({"backward": backward}), flush=True)
            return 0
    wall_ms, kern_ms, extra, (o_dev, lse_dev) = time_workload(wl, args.steps, args.warmup, tiles)
    value = wl.flops / (wall_ms * 1e-3) / 1e12
    achieved = wl.flops / (kern_ms * 1e-3) / 1e12
    print(f"[bench] {wl.name}: {wall_ms:.4f} ms/step, kernel {kern_ms:.4f} ms, {value:.1f} TFLOP/s",
          file=sys.stderr, flush=True)

    sweep = {}
    if not args.no_sweep:
        from exact_tiled_attention_07_amd.inputs import Workload

        # the metric's range of T at B4 H12 d64 causal: the workloads at T = 1024 and 16384, two
        # points in between (seeded like the others), and the d = 128 workload with its causal variant
        between = {"t2048": Workload("t2048_causal_B4_H12_T2048_d64", 4, 12, 2048, 64, True, seed=7),
                   "t8192": Workload("t8192_causal_B4_H12_T8192_d64", 4, 12, 8192, 64, True, seed=8),
                   "c5b_causal": Workload("c5b_causal_B4_H16_T8192_d128", 4, 16, 8192, 128, True, seed=9)}
        for name in ("c3", "t2048", "c4", "t8192", "c5a", "c5b", "c5b_causal"):
            if name == args.workload:
                continue
            w2 = between[name] if name in between else WORKLOADS[name]
            # short launches get more steps, so warm-up and timing each span about 25 ms of work
            # (the shader clock rises over the first milliseconds of load)
            est_s = w2.flops / 800e12
            n_t = min(2000, max(5, args.steps // 5, math.ceil(0.025 / est_s)))
            n_w = min(2000, max(2, args.warmup // 5, math.ceil(0.025 / est_s)))
            wms, kms, ex2, _ = time_workload(w2, n_t, n_w, None)
            sweep[name] = {"workload": w2.name, "ms_per_step": round(wms, 5),
                           "tflops": round(w2.flops / (wms * 1e-3) / 1e12, 2),
                           "kernel_tflops": round(w2.flops / (kms * 1e-3) / 1e12, 2),
                           "pct_of_peak": round(100 * w2.flops / (kms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}
            print(f"[bench] sweep {w2.name}: {sweep[name]}", file=sys.stderr, flush=True)

    sparse = None
    if not args.no_sparse:
        sparse = time_sparse(WORKLOADS["c5a"], max(5, args.steps // 10), max(2, args.warmup // 10))
        print(f"[bench] sparse: {sparse}", file=sys.stderr, flush=True)

    splitkv = None
    if not args.no_splitkv:
        splitkv = time_splitkv(args.steps, args.warmup)
        print(f"[bench] splitkv: {splitkv}", file=sys.stderr, flush=True)

    fp8 = None
    if not args.no_fp8:
        fp8 = time_fp8(("c4", "c5a", "c5b"), args.steps, args.warmup)
        print(f"[bench] fp8: {fp8}", file=sys.stderr, flush=True)

    copy_calibration(args.copy_calibration_mib)

    base = parity = None
    if not args.no_cpu_baseline:
        base, ref, n_heads = cpu_baseline(wl)
        print(f"[bench] cpu baseline: {base}", file=sys.stderr, flush=True)
        parity = parity_check(wl, o_dev, lse_dev, ref, n_heads)
        print(f"[bench] parity: {parity}", file=sys.stderr, flush=True)
        del ref
        # every workload (the bench's own workload is the object above)
        base["per_config"] = cpu_baseline_per_config(tuple(n for n in PER_CONFIG if n != args.workload))
        print(f"[bench] cpu baseline per config: {base['per_config']}", file=sys.stderr, flush=True)

    profiled = args.workload == PROFILED_WORKLOAD and tiles is None
    traffic = recorded_traffic() if profiled else None
    clock = recorded_clock_mhz() if profiled else None
    peak_at_clock = MFMA_FLOP_PER_CLK * clock * 1e6 / 1e12 if clock else None
    line = {
        "metric": "causal attn fwd TFLOP/s & % of bf16 MFMA peak, B4 H12 d64, T=1K..16K",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normal draws times config.input_sigma, rounded to bf16)",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "T": wl.T, "d": wl.d,
                   "causal": wl.causal, "input_sigma": wl.sigma, "scale": wl.scale,
                   "tiles": args.tiles or "default"},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel_ms": round(kern_ms, 5),
                     "clock_mhz": clock,
                     "peak_at_clock": round(peak_at_clock, 1) if peak_at_clock else None,
                     "frac_at_clock": round(achieved / peak_at_clock, 4) if peak_at_clock else None,
                     "timing": "achieved = flops per launch / (one HIP event pair on the launch stream "
                               "around the timed launches / steps)",
                     "flops_per_launch": wl.flops,
                     "compulsory_bytes": compulsory_bytes(wl),
                     "compulsory_gbs": round(compulsory_bytes(wl) / (kern_ms * 1e-3) / 1e9, 1),
                     **extra},
        "cpu_baseline": base,
        "parity": parity,
        "sweep": sweep,
        "backward": backward,
        "sparse": sparse,
        "splitkv": splitkv,
        "fp8": fp8,
        "context": {"note": "claims printed on the source pages about other GPUs; not targets",
                    "claims": PAGE_CLAIMS},
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

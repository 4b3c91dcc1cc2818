"""Seeded synthetic inputs for exact attention forward.

This module holds no attention arithmetic. It only draws numbers and rounds them to bf16, so the
CPU oracle and the GPU path can both be fed the very same bits.

Recipe: numpy ``Generator(PCG64(seed))`` draws ``standard_normal`` float32 arrays of shape
``[B, H, T, d]`` in the order q, k, v. Each array is multiplied by ``sigma`` in float32 and rounded
to bf16 with round-to-nearest-even. The workloads are the causal bf16 forward at batch 4, 12 heads,
head_dim 64 for T from 512 to 16,384, and the ragged T=1000 check at batch 2
(learn-llm.fim.ai "手写 FlashAttention：拆开 SDPA 这个黑盒", the setup line above STEP 1, and
STEP 4's error-check note).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


def bf16_bits_from_f32(x) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return the uint16 bits."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    nan = np.isnan(a)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    # keep NaN a quiet NaN (the rounding add could otherwise carry it into an infinity)
    rounded[nan] = ((u[nan] >> 16).astype(np.uint16) | np.uint16(0x0040))
    return rounded.reshape(a.shape)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32).reshape(b.shape)


def make_qkv(B: int, H: int, T: int, d: int, seed: int, sigma: float = 1.0):
    """Draw q, k, v as bf16 bit patterns ``[B, H, T, d]`` from ``Generator(PCG64(seed))``."""
    gen = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(3):  # order: q, k, v
        x = gen.standard_normal((B, H, T, d), dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        out.append(bf16_bits_from_f32(x))
    return tuple(out)


def sparse_mask(T: int, density: float, seed: int) -> np.ndarray:
    """A block mask for the block-sparse forward, uint8 [1, ceil(T/128), ceil(T/64)] (one mask for
    every head): each 128 x 64 block kept when a PCG64(seed) uniform draw is below `density`, plus
    the two blocks on each query block's diagonal, so that every query sees a key."""
    nq, nk = -(-T // 128), -(-T // 64)
    m = (np.random.Generator(np.random.PCG64(seed)).random((1, nq, nk)) < density).astype(np.uint8)
    for i in range(nq):
        m[0, i, 2 * i:min(nk, 2 * i + 2)] = 1
    return m


def to_torch_bf16(bits, device="cpu"):
    """View uint16 bf16 bit patterns as a torch bfloat16 tensor on ``device`` (no rounding)."""
    import torch

    arr = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
    return t.to(device)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    d: int
    causal: bool
    seed: int
    sigma: float = 1.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def flops(self) -> float:
        """Counted flops: 2*B*H*T^2*d causal (the visible half), 4*B*H*T^2*d otherwise."""
        f = 2.0 * self.B * self.H * self.T * self.T * self.d
        return f if self.causal else 2.0 * f

    def make(self):
        return make_qkv(self.B, self.H, self.T, self.d, self.seed, self.sigma)


# The five workloads (the fifth has a causal d=64 part and a non-causal d=128 part).
WORKLOADS = {
    "c1": Workload("c1_causal_B1_H2_T256_d64", 1, 2, 256, 64, True, seed=1),
    "c2": Workload("c2_causal_B2_H12_T1000_d64", 2, 12, 1000, 64, True, seed=2),
    "c3": Workload("c3_causal_B4_H12_T1024_d64", 4, 12, 1024, 64, True, seed=3),
    "c4": Workload("c4_causal_B4_H12_T4096_d64_x2", 4, 12, 4096, 64, True, seed=4, sigma=2.0),
    "c5a": Workload("c5a_causal_B4_H12_T16384_d64", 4, 12, 16384, 64, True, seed=5),
    "c5b": Workload("c5b_noncausal_B4_H16_T8192_d128", 4, 16, 8192, 128, False, seed=6),
}


def make_partials(n: int, B: int, H: int, T: int, d: int, seed: int, lse_sigma: float = 4.0,
                  p_empty: float = 0.1):
    """Draw synthetic partial results for a merge: ``o_parts`` float32 ``[n, B, H, T, d]`` and
    ``lse_parts`` float32 ``[n, B, H, T]`` from ``Generator(PCG64(seed))`` (o, then lse, then the
    empty flags). A fraction ``p_empty`` of the parts is empty: LSE = -inf and O = 0."""
    gen = np.random.Generator(np.random.PCG64(seed))
    o = gen.standard_normal((n, B, H, T, d), dtype=np.float32)
    lse = gen.standard_normal((n, B, H, T), dtype=np.float32) * np.float32(lse_sigma)
    empty = gen.random((n, B, H, T)) < p_empty
    lse[empty] = -np.inf
    o[empty] = 0.0
    return o, lse


def quantize_e4m3(x, descale: float):
    """FP8 E4M3 (OCP, no infinities) codes of ``x / descale``: round to nearest even, values beyond
    the largest finite magnitude (448) clamped to it. Returns uint8 codes."""
    import torch

    y = np.clip(np.asarray(x, dtype=np.float32) / np.float32(descale), -448.0, 448.0)
    return torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def make_qkv_fp8(B: int, H: int, T: int, d: int, seed: int, sigma: float = 1.0):
    """FP8 inputs: ``make_qkv``'s normal draws (same generator, same order, times sigma) quantized per
    tensor to E4M3 with the descale factor amax / 448 (in float32), so the largest magnitude of each
    tensor maps to the largest code. Returns ``(q8, k8, v8, (q_descale, k_descale, v_descale))``."""
    gen = np.random.Generator(np.random.PCG64(seed))
    codes, scales = [], []
    for _ in range(3):  # order: q, k, v
        x = gen.standard_normal((B, H, T, d), dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        amax = float(np.abs(x).max()) if x.size else 1.0
        descale = float(np.float32(max(amax, 1e-30) / 448.0))
        codes.append(quantize_e4m3(x, descale))
        scales.append(descale)
    return codes[0], codes[1], codes[2], tuple(scales)

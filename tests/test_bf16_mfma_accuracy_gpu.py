"""Accuracy of the bf16 matrix instruction that the forward uses, measured on the device.

tests/bf16_mfma_probe.hip chains v_mfma_f32_32x32x16_bf16 over k in one fp32 accumulator, as the
forward does for the scores (k = d) and for P V (k = the keys, 64 per tile and every tile of a row
into the same accumulator). Each of its 32 x 32 outputs is compared with the exact dot product (a
product of two bf16 values has at most 16 significant bits, so it is exact in float64, and so are
the float64 sums checked here to far below fp32's precision).

The bounds checked are those of the bf16 forward's derived element bound (tests/fwd_bounds.py): for
the long P V chains the textbook one for a recursive fp32 sum of k terms with each addition rounded
once, toward zero or to nearest, |c - sum_k a_k b_k| <= k 2^-23 sum_k |a_k b_k| (EPS_BF16_SUM); for
the score chains over the head dimension (k = 64, 128) 2^-22 sum_k |a_k b_k| (EPS_BF16_QK), which
the instruction meets with room (measured 9.2e-8: it adds like fp32 rounded to nearest, unlike the
FP8 instruction, which truncates).
"""
import ctypes
import os

import numpy as np
import pytest
import torch

from exact_tiled_attention_07_amd.inputs import bf16_bits_from_f32, bf16_bits_to_f32, make_qkv
from fwd_bounds import EPS_BF16_QK, EPS_BF16_SUM

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
PROBE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbf16_mfma_probe.so")


def probe(a_bits, b_bits):
    """c[g] = A[g] B[g]^T on the device; a_bits, b_bits uint16 (bf16) [n, 32, k]."""
    assert os.path.exists(PROBE), f"{PROBE} is not built (__graft_entry__.build())"
    lib = ctypes.CDLL(PROBE)
    lib.bf16_mfma_probe.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.bf16_mfma_probe.restype = ctypes.c_int
    n, rows, k = a_bits.shape
    assert rows == 32 and b_bits.shape == a_bits.shape
    a = torch.from_numpy(np.ascontiguousarray(a_bits).view(np.int16)).to(DEV)
    b = torch.from_numpy(np.ascontiguousarray(b_bits).view(np.int16)).to(DEV)
    c = torch.full((n, 32, 32), float("nan"), dtype=torch.float32, device=DEV)
    rc = lib.bf16_mfma_probe(a.data_ptr(), b.data_ptr(), c.data_ptr(), n, k,
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    return c.cpu().numpy().astype(np.float64)


def relative_errors(a_bits, b_bits, c):
    a, b = (bf16_bits_to_f32(x).astype(np.float64) for x in (a_bits, b_bits))
    exact = np.einsum("gik,gjk->gij", a, b)
    mag = np.einsum("gik,gjk->gij", np.abs(a), np.abs(b))
    err = np.abs(c - exact)
    return np.where(mag > 0, err / np.where(mag > 0, mag, 1.0), err)


def report(label, k, rel):
    print(f"[gpu bf16 mfma] {label}, k={k}: {rel.size} outputs, max error / sum|ab| = {rel.max():.3e} "
          f"({rel.max() / (k * 2.0 ** -23):.2e} of k 2^-23)", flush=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("sigma", [1.0, 2.0, 4.0])
def test_scores(d, sigma):
    # Q K^T blocks: 32 key rows against 32 query rows over the head dimension, as the score MFMAs
    qb, kb, _ = make_qkv(1, 2, 4096, d, seed=31, sigma=sigma)
    a, b = kb.reshape(-1, 32, d), qb.reshape(-1, 32, d)
    rel = relative_errors(a, b, probe(a, b))
    report(f"scores, N(0, {sigma}^2) rows", d, rel)
    assert rel.max() <= EPS_BF16_QK


@pytest.mark.parametrize("keys", [64, 1024, 16384])
@pytest.mark.parametrize("sigma,scale", [(1.0, 0.125), (2.0, 0.125), (1.0, 0.01)])
def test_weights_times_values(keys, sigma, scale):
    # P V over a row's keys: the weights exp(s - m) of 32 queries (m the max over the keys shown),
    # rounded to bf16, against 32 channels of those keys' values, accumulated over every key
    n_q = 32 * max(1, 4096 // keys)
    qb, kb, vb = make_qkv(1, 1, max(keys, n_q), 64, seed=41, sigma=sigma)
    q, k, v = (bf16_bits_to_f32(x)[0, 0].astype(np.float64) for x in (qb, kb, vb))
    s = (q[:n_q] @ k[:keys].T) * scale
    w = np.exp(s - s.max(axis=1, keepdims=True))
    p_bits = bf16_bits_from_f32(w.astype(np.float32))                # [n_q, keys]
    vt_bits = np.ascontiguousarray(vb[0, 0, :keys, :32].T)           # V^T: 32 channels x keys
    a = np.broadcast_to(vt_bits, (n_q // 32, 32, keys)).copy()
    b = p_bits.reshape(n_q // 32, 32, keys)
    rel = relative_errors(a, b, probe(a, b))
    report(f"P V, N(0, {sigma}^2), scale {scale}", keys, rel)
    assert rel.max() <= EPS_BF16_SUM * keys

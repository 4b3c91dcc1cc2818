"""CPU oracle for exact attention, forward and backward — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package. The GPU library never imports, links or calls it, and this package imports nothing
from the GPU package: the two share only the seeded input generator, which holds none of the
method's arithmetic.

The arithmetic lives in ``fa_ref.c`` (plain C, double precision, OpenMP over rows). It is the
naive, two-pass definition of attention on the bf16 inputs:

* scores ``S = scale * Q K^T``, a row softmax, then ``P V`` (learn-llm.fim.ai
  "手写 FlashAttention：拆开 SDPA 这个黑盒", STEP 1);
* the row maximum is subtracted before ``exp`` (same page, STEP 2);
* with a causal mask only keys ``j <= i`` are visible to query ``i`` (same page, STEP 3);
* the natural-log logsumexp of each row's visible scaled scores is returned alongside ``O``
  (same page, STEP 4, the note on what the forward saves for the backward).

``fa_ref_bwd.c`` holds the backward: the gradients of that forward with respect to ``Q``, ``K``
and ``V`` for an output gradient ``dO``, with the probabilities recomputed from ``Q`` and ``K``
(same page, STEP 4, the note on training; ijyty.com FlashAttention article, section 2.2), plus a
float64-input forward with the same order of operations for finite-difference checks.

``fa_ref_sparse.c`` holds the block-sparse forward: keys of a (query block, key block) whose mask
is zero are not visible, the way the causal mask hides the blocks above the diagonal (cnblogs
"内核案例研究：Flash Attention", section "块稀疏注意力 V2 和 V3"); a row with no visible key gets
``O = 0`` and ``LSE = -inf``.

Three functions are numpy float64 rather than C: ``merge_partials``, the log-space combine of
partial results over disjoint key ranges (ijyty.com FlashAttention article, section 2.1),
``attention_fwd_cross``, the plain two-pass attention of T queries over a key range of a Tk-key
sequence (one library matmul per head for the scores and one for P V), and ``attention_bwd_rows``,
the backward's definitions evaluated for selected query and key rows of long heads.

``attention_fwd_fp8`` decodes FP8 E4M3 codes exactly, applies the per-tensor descale factors in
float64 and calls the float64 forward; ``attention_fwd_fp8_rows`` evaluates the same definition in
numpy for selected rows of long heads.

Every function here is pinned by the ``not gpu`` tests in ``tests/test_oracle_pins.py``,
``tests/test_oracle_bwd_pins.py``, ``tests/test_oracle_sparse_pins.py``,
``tests/test_oracle_splitkv_pins.py`` and ``tests/test_oracle_fp8_pins.py`` against closed forms, invariants, finite differences, brute
force and library special cases.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_ref.c")
_SRC_BWD = os.path.join(_HERE, "fa_ref_bwd.c")
_SRC_SPARSE = os.path.join(_HERE, "fa_ref_sparse.c")
# FA_ORACLE_LIB names another build of the same sources (the sanitizer test loads an ASan/UBSan one)
_LIB_PATH = os.environ.get("FA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``fa_ref.c`` into ``liboracle.so`` next to it (gcc, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
               "-Wall", "-Wextra", "-o", tmp, _SRC, _SRC_BWD, _SRC_SPARSE, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    p_u16 = ctypes.POINTER(ctypes.c_uint16)
    p_f64 = ctypes.POINTER(ctypes.c_double)
    p_i64 = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.fa_ref_fwd.argtypes = [p_u16, p_u16, p_u16, p_f64, p_f64, i64, i64, i64, i64,
                               ctypes.c_int, ctypes.c_double, ctypes.c_int]
    lib.fa_ref_fwd.restype = ctypes.c_int
    lib.fa_ref_fwd_rows.argtypes = [p_u16, p_u16, p_u16, i64, i64, i64, i64, ctypes.c_int,
                                    ctypes.c_double, p_i64, i64, p_f64, p_f64, ctypes.c_int]
    lib.fa_ref_fwd_rows.restype = ctypes.c_int
    lib.fa_ref_threads_used.argtypes = [ctypes.c_int]
    lib.fa_ref_threads_used.restype = ctypes.c_int
    lib.fa_ref_fwd_f64.argtypes = [p_f64, p_f64, p_f64, p_f64, p_f64, i64, i64, i64, i64,
                                   ctypes.c_int, ctypes.c_double, ctypes.c_int]
    lib.fa_ref_fwd_f64.restype = ctypes.c_int
    lib.fa_ref_bwd_f64.argtypes = [p_f64, p_f64, p_f64, p_f64, p_f64, p_f64, p_f64, p_f64, i64, i64,
                                   i64, i64, ctypes.c_int, ctypes.c_double, ctypes.c_int]
    lib.fa_ref_bwd_f64.restype = ctypes.c_int
    lib.fa_ref_bwd.argtypes = [p_u16, p_u16, p_u16, p_u16, p_f64, p_f64, p_f64, p_f64, i64, i64, i64,
                               i64, ctypes.c_int, ctypes.c_double, ctypes.c_int]
    lib.fa_ref_bwd.restype = ctypes.c_int
    lib.fa_ref_fwd_blockmask.argtypes = [p_u16, p_u16, p_u16, p_f64, p_f64, i64, i64, i64, i64,
                                         ctypes.c_int, ctypes.c_double,
                                         ctypes.POINTER(ctypes.c_uint8), i64, i64, i64, ctypes.c_int]
    lib.fa_ref_fwd_blockmask.restype = ctypes.c_int
    _lib = lib
    return lib


def _as_bf16_bits(x: np.ndarray, name: str) -> np.ndarray:
    if x.dtype != np.uint16:
        raise TypeError(f"{name}: expected bf16 bit patterns as uint16, got {x.dtype}")
    if x.ndim != 4:
        raise ValueError(f"{name}: expected [B, H, T, d], got shape {x.shape}")
    return np.ascontiguousarray(x)


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def threads_used(num_threads: int = 0) -> int:
    """Threads an OpenMP team of the oracle actually gets for ``num_threads`` (0: default)."""
    return int(_load().fa_ref_threads_used(int(num_threads)))


def attention_fwd(q_bits, k_bits, v_bits, causal: bool, scale: float, num_threads: int = 0):
    """Exact attention forward on bf16 inputs given as uint16 bit patterns ``[B, H, T, d]``.

    Returns ``(o, lse)``: ``o`` float64 ``[B, H, T, d]`` and ``lse`` float64 ``[B, H, T]``
    (natural log of the row's sum of ``exp`` over the visible scaled scores).
    """
    q = _as_bf16_bits(q_bits, "q")
    k = _as_bf16_bits(k_bits, "k")
    v = _as_bf16_bits(v_bits, "v")
    if not (q.shape == k.shape == v.shape):
        raise ValueError(f"q/k/v shapes differ: {q.shape} {k.shape} {v.shape}")
    B, H, T, d = q.shape
    o = np.empty((B, H, T, d), dtype=np.float64)
    lse = np.empty((B, H, T), dtype=np.float64)
    rc = _load().fa_ref_fwd(_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                            _ptr(v, ctypes.c_uint16), _ptr(o, ctypes.c_double),
                            _ptr(lse, ctypes.c_double), B, H, T, d, int(bool(causal)),
                            float(scale), int(num_threads))
    if rc != 0:
        raise RuntimeError(f"fa_ref_fwd failed with code {rc}")
    return o, lse


def attention_rows(q_bits, k_bits, v_bits, causal: bool, scale: float, rows, num_threads: int = 0):
    """Exact attention forward for selected rows only.

    ``rows`` holds flat row indices ``(b*H + h)*T + i``. Returns ``(o, lse)`` with ``o`` float64
    ``[len(rows), d]`` and ``lse`` float64 ``[len(rows)]``.
    """
    q = _as_bf16_bits(q_bits, "q")
    k = _as_bf16_bits(k_bits, "k")
    v = _as_bf16_bits(v_bits, "v")
    if not (q.shape == k.shape == v.shape):
        raise ValueError(f"q/k/v shapes differ: {q.shape} {k.shape} {v.shape}")
    B, H, T, d = q.shape
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    o = np.empty((r.size, d), dtype=np.float64)
    lse = np.empty((r.size,), dtype=np.float64)
    rc = _load().fa_ref_fwd_rows(_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                                 _ptr(v, ctypes.c_uint16), B, H, T, d, int(bool(causal)),
                                 float(scale), _ptr(r, ctypes.c_int64), r.size,
                                 _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double),
                                 int(num_threads))
    if rc != 0:
        raise RuntimeError(f"fa_ref_fwd_rows failed with code {rc}")
    return o, lse


def _as_f64(x, name: str) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if a.ndim != 4:
        raise ValueError(f"{name}: expected [B, H, T, d], got shape {a.shape}")
    return a


def attention_fwd_f64(q, k, v, causal: bool, scale: float, num_threads: int = 0):
    """The forward on float64 inputs, in the same order of operations as ``attention_fwd``.

    For checking the backward against finite differences of the forward. Returns ``(o, lse)``.
    """
    q, k, v = _as_f64(q, "q"), _as_f64(k, "k"), _as_f64(v, "v")
    if not (q.shape == k.shape == v.shape):
        raise ValueError(f"q/k/v shapes differ: {q.shape} {k.shape} {v.shape}")
    B, H, T, d = q.shape
    o = np.empty((B, H, T, d), dtype=np.float64)
    lse = np.empty((B, H, T), dtype=np.float64)
    rc = _load().fa_ref_fwd_f64(_ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double),
                                _ptr(v, ctypes.c_double), _ptr(o, ctypes.c_double),
                                _ptr(lse, ctypes.c_double), B, H, T, d, int(bool(causal)),
                                float(scale), int(num_threads))
    if rc != 0:
        raise RuntimeError(f"fa_ref_fwd_f64 failed with code {rc}")
    return o, lse


def _bwd_out(shape):
    B, H, T, d = shape
    return (np.empty(shape, dtype=np.float64), np.empty(shape, dtype=np.float64),
            np.empty(shape, dtype=np.float64), np.empty((B, H, T), dtype=np.float64))


def attention_bwd(q_bits, k_bits, v_bits, do_bits, causal: bool, scale: float, num_threads: int = 0):
    """Exact attention backward on bf16 inputs (uint16 bit patterns ``[B, H, T, d]``).

    ``do_bits`` is the output gradient. The probabilities are recomputed from ``q`` and ``k`` in
    float64 (nothing from a forward run is taken). Returns ``(dq, dk, dv, delta)``: float64
    gradients ``[B, H, T, d]`` and ``delta[b, h, i] = dO_i . O_i`` ``[B, H, T]``.
    """
    q, k = _as_bf16_bits(q_bits, "q"), _as_bf16_bits(k_bits, "k")
    v, do = _as_bf16_bits(v_bits, "v"), _as_bf16_bits(do_bits, "do")
    if not (q.shape == k.shape == v.shape == do.shape):
        raise ValueError(f"q/k/v/do shapes differ: {q.shape} {k.shape} {v.shape} {do.shape}")
    B, H, T, d = q.shape
    dq, dk, dv, delta = _bwd_out(q.shape)
    rc = _load().fa_ref_bwd(_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                            _ptr(v, ctypes.c_uint16), _ptr(do, ctypes.c_uint16),
                            _ptr(dq, ctypes.c_double), _ptr(dk, ctypes.c_double),
                            _ptr(dv, ctypes.c_double), _ptr(delta, ctypes.c_double),
                            B, H, T, d, int(bool(causal)), float(scale), int(num_threads))
    if rc != 0:
        raise RuntimeError(f"fa_ref_bwd failed with code {rc}")
    return dq, dk, dv, delta


def attention_bwd_f64(q, k, v, do, causal: bool, scale: float, num_threads: int = 0):
    """The backward on float64 inputs (for finite-difference and library checks)."""
    q, k, v, do = _as_f64(q, "q"), _as_f64(k, "k"), _as_f64(v, "v"), _as_f64(do, "do")
    if not (q.shape == k.shape == v.shape == do.shape):
        raise ValueError(f"q/k/v/do shapes differ: {q.shape} {k.shape} {v.shape} {do.shape}")
    B, H, T, d = q.shape
    dq, dk, dv, delta = _bwd_out(q.shape)
    rc = _load().fa_ref_bwd_f64(_ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double),
                                _ptr(v, ctypes.c_double), _ptr(do, ctypes.c_double),
                                _ptr(dq, ctypes.c_double), _ptr(dk, ctypes.c_double),
                                _ptr(dv, ctypes.c_double), _ptr(delta, ctypes.c_double),
                                B, H, T, d, int(bool(causal)), float(scale), int(num_threads))
    if rc != 0:
        raise RuntimeError(f"fa_ref_bwd_f64 failed with code {rc}")
    return dq, dk, dv, delta


def attention_bwd_rows(q_bits, k_bits, v_bits, do_bits, causal: bool, scale: float, q_rows, k_rows,
                       block_rows: int = 512):
    """The backward for selected rows, in numpy float64, for heads too long for ``attention_bwd``.

    ``q_rows`` and ``k_rows`` are flat row indices ``(b*H + h)*T + i``. Returns ``(dq, dk, dv,
    delta)``: ``dq`` float64 ``[len(q_rows), d]`` (gradient of query row i), ``dk`` and ``dv``
    ``[len(k_rows), d]`` (gradients of key/value row j), and ``delta`` ``[len(q_rows)]``
    (``D_i = dO_i . O_i``). The same definitions as ``attention_bwd`` (learn-llm.fim.ai
    "手写 FlashAttention：拆开 SDPA 这个黑盒", STEP 4; ijyty.com FlashAttention article, section
    2.2), evaluated row by row: for each head that a requested row belongs to, every query row's
    LSE_i and D_i come from its own two-pass softmax (rows taken a block at a time only to bound
    memory), then
        P_ij = exp(scale q_i.k_j - LSE_i),  dP_ij = dO_i.v_j,  dS_ij = P_ij (dP_ij - D_i),
        dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i
    over the visible pairs (j <= i when causal).
    """
    q, k = _bf16_to_f64(_as_bf16_bits(q_bits, "q")), _bf16_to_f64(_as_bf16_bits(k_bits, "k"))
    v, do = _bf16_to_f64(_as_bf16_bits(v_bits, "v")), _bf16_to_f64(_as_bf16_bits(do_bits, "do"))
    if not (q.shape == k.shape == v.shape == do.shape):
        raise ValueError(f"q/k/v/do shapes differ: {q.shape} {k.shape} {v.shape} {do.shape}")
    B, H, T, d = q.shape
    qr = np.asarray(q_rows, dtype=np.int64).reshape(-1)
    kr = np.asarray(k_rows, dtype=np.int64).reshape(-1)
    dq = np.empty((qr.size, d)); dk = np.empty((kr.size, d)); dv = np.empty((kr.size, d))
    delta = np.empty(qr.size)
    idx = np.arange(T)
    for head in sorted(set((qr // T).tolist()) | set((kr // T).tolist())):
        b, h = divmod(head, H)
        Q, K, V, dO = q[b, h], k[b, h], v[b, h], do[b, h]
        lse, D = np.empty(T), np.empty(T)
        for i0 in range(0, T, block_rows):
            i1 = min(i0 + block_rows, T)
            kend = i1 if causal else T  # keys past the block's last row are hidden from all of it
            s = scale * (Q[i0:i1] @ K[:kend].T)
            if causal:
                s = np.where(idx[None, :kend] > idx[i0:i1, None], -np.inf, s)
            m = s.max(axis=1)
            e = np.exp(s - m[:, None])
            l = e.sum(axis=1)
            o = (e @ V[:kend]) / l[:, None]
            lse[i0:i1] = m + np.log(l)
            D[i0:i1] = (dO[i0:i1] * o).sum(axis=1)
        for n in np.nonzero(qr // T == head)[0]:
            i = int(qr[n] % T)
            vis = idx <= i if causal else np.ones(T, dtype=bool)
            p = np.exp(scale * (K[vis] @ Q[i]) - lse[i])
            ds = p * (V[vis] @ dO[i] - D[i])
            dq[n] = scale * (ds @ K[vis])
            delta[n] = D[i]
        for n in np.nonzero(kr // T == head)[0]:
            j = int(kr[n] % T)
            vis = idx >= j if causal else np.ones(T, dtype=bool)
            p = np.exp(scale * (Q[vis] @ K[j]) - lse[vis])
            dv[n] = p @ dO[vis]
            ds = p * (dO[vis] @ V[j] - D[vis])
            dk[n] = scale * (ds @ Q[vis])
    return dq, dk, dv, delta


def attention_fwd_blockmask(q_bits, k_bits, v_bits, causal: bool, scale: float, mask,
                            block_m: int, block_n: int, num_threads: int = 0):
    """Block-sparse attention forward on bf16 inputs.

    ``mask`` is uint8 ``[mask_heads, ceil(T/block_m), ceil(T/block_n)]`` with ``mask_heads`` 1 or
    ``B*H``; key j is visible to query i iff the mask of (i // block_m, j // block_n) is nonzero
    (and j <= i when causal). Rows with no visible key get ``O = 0``, ``LSE = -inf``.
    """
    q, k, v = _as_bf16_bits(q_bits, "q"), _as_bf16_bits(k_bits, "k"), _as_bf16_bits(v_bits, "v")
    if not (q.shape == k.shape == v.shape):
        raise ValueError(f"q/k/v shapes differ: {q.shape} {k.shape} {v.shape}")
    B, H, T, d = q.shape
    m = np.ascontiguousarray(np.asarray(mask, dtype=np.uint8))
    nqb, nkb = -(-T // block_m), -(-T // block_n)
    if m.ndim != 3 or m.shape[1:] != (nqb, nkb) or m.shape[0] not in (1, B * H):
        raise ValueError(f"mask must be [1 or B*H, {nqb}, {nkb}], got {m.shape}")
    o = np.empty((B, H, T, d), dtype=np.float64)
    lse = np.empty((B, H, T), dtype=np.float64)
    rc = _load().fa_ref_fwd_blockmask(_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                                      _ptr(v, ctypes.c_uint16), _ptr(o, ctypes.c_double),
                                      _ptr(lse, ctypes.c_double), B, H, T, d, int(bool(causal)),
                                      float(scale), _ptr(m, ctypes.c_uint8), m.shape[0], block_m,
                                      block_n, int(num_threads))
    if rc != 0:
        raise RuntimeError(f"fa_ref_fwd_blockmask failed with code {rc}")
    return o, lse


def merge_partials(o_parts, lse_parts):
    """Log-space combine of partial results over disjoint key ranges, in float64.

    ``LSE = log sum_s exp(LSE_s)`` and ``O = sum_s exp(LSE_s - LSE) O_s`` (ijyty.com FlashAttention
    article, section 2.1: the per-block logsumexp accumulated in log space and the output divided by
    exp(lse) at the end). Parts with LSE_s = -inf contribute nothing; rows whose parts are all -inf
    get O = 0 and LSE = -inf. ``o_parts`` ``[n, ..., d]``, ``lse_parts`` ``[n, ...]``.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(lse_parts - m_safe[None])          # exp(-inf) = 0 for empty parts
    l = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        o = (w[..., None] * o_parts).sum(axis=0) / np.where(empty, 1.0, l)[..., None]
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    o[empty] = 0.0
    return o, lse


def attention_fwd_key_range(q_bits, k_bits, v_bits, causal: bool, scale: float, k_begin: int,
                            k_end: int, num_threads: int = 0):
    """Attention of every query over the keys [k_begin, k_end) only (k_begin a multiple of 64, k_end
    a multiple of 64 or T): the block-sparse oracle with one query block and the range's 64-key
    blocks. Returns ``(o, lse)`` float64; rows with no visible key get 0 and -inf."""
    T = q_bits.shape[2]
    nk = -(-T // 64)
    mask = np.zeros((1, 1, nk), dtype=np.uint8)
    mask[0, 0, k_begin // 64:-(-k_end // 64)] = 1
    return attention_fwd_blockmask(q_bits, k_bits, v_bits, causal, scale, mask, max(T, 1), 64,
                                   num_threads)


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64, exactly (a bf16 value is the top half of a float32)."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def attention_fwd_cross(q_bits, k_bits, v_bits, causal: bool, scale: float, k_begin: int = 0,
                        k_end: int | None = None):
    """Exact attention of T queries over the keys [k_begin, k_end) of a sequence of Tk keys, in
    float64 with numpy (q ``[B, H, T, d]``, k and v ``[B, H, Tk, d]``, bf16 bit patterns).

    The plain two-pass definition, as in ``fa_ref.c``, for every row: the scores ``scale * q_i . k_j``
    of the visible keys, their maximum, the exponentials and their sum, then ``O = sum e_j v_j / l``
    and ``LSE = m + ln l``. With the causal mask the queries are the last T positions of the keys'
    sequence (keys held for earlier positions, as when decoding after a prefix), so query i sees
    key j iff ``j <= i + Tk - T``; the pages treat only T = Tk, where this is the usual ``j <= i``
    (learn-llm.fim.ai "手写 FlashAttention：拆开 SDPA 这个黑盒", STEP 3). A row with no visible key
    gets ``O = 0`` and ``LSE = -inf``. Returns ``(o, lse)`` float64.
    """
    q = _as_bf16_bits(q_bits, "q")
    k = _as_bf16_bits(k_bits, "k")
    v = _as_bf16_bits(v_bits, "v")
    B, H, T, d = q.shape
    Tk = k.shape[2]
    if k.shape != v.shape or k.shape[:2] != (B, H) or k.shape[3] != d:
        raise ValueError(f"k, v must be [B, H, Tk, d] like q: {q.shape} {k.shape} {v.shape}")
    k_end = Tk if k_end is None else k_end
    if not (0 <= k_begin <= k_end <= Tk):
        raise ValueError(f"key range [{k_begin}, {k_end}) outside [0, {Tk})")
    j = np.arange(Tk)[None, :]
    i = np.arange(T)[:, None]
    visible = (j >= k_begin) & (j < k_end)
    if causal:
        visible = visible & (j <= i + (Tk - T))
    o = np.zeros((B, H, T, d))
    lse = np.full((B, H, T), -np.inf)
    has_key = visible.any(axis=1)
    for b in range(B):
        for h in range(H):
            qf, kf, vf = (_bf16_to_f64(x[b, h]) for x in (q, k, v))
            s = float(scale) * (qf @ kf.T)
            s = np.where(visible, s, -np.inf)
            m = s.max(axis=1, initial=-np.inf)
            m_safe = np.where(has_key, m, 0.0)
            e = np.exp(s - m_safe[:, None])            # exp(-inf) = 0 for hidden keys
            l = e.sum(axis=1)
            l_safe = np.where(has_key, l, 1.0)
            o[b, h] = np.where(has_key[:, None], (e @ vf) / l_safe[:, None], 0.0)
            lse[b, h] = np.where(has_key, m_safe + np.log(l_safe), -np.inf)
    return o, lse


def e4m3_to_f64(codes) -> np.ndarray:
    """Decode OCP FP8 E4M3 codes (uint8) to float64, exactly.

    The format (the OCP 8-bit floating point specification's E4M3, the "fn" variant with no
    infinities): sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is subnormal
    (m * 2^-9); S.1111.111 is NaN; the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, out)


def attention_fwd_fp8(q8, k8, v8, causal: bool, scale: float, q_descale: float, k_descale: float,
                      v_descale: float, num_threads: int = 0):
    """Exact attention on FP8 inputs: the inputs are the E4M3 codes times their per-tensor descale
    factors (``q = e4m3(q8) * q_descale``, likewise k and v), and the result is the exact attention of
    those values in float64 (``attention_fwd_f64``).

    Low-precision inputs that double the matrix throughput are the pages' next step (cnblogs
    "内核案例研究：Flash Attention", the closing section on V3: FP8 on Hopper); the decode and the
    descale are exact in float64 (a 4-bit significand times an fp32 factor), so this is the plain
    definition on the values the codes stand for. Returns ``(o, lse)`` float64.
    """
    for name, x in (("q8", q8), ("k8", k8), ("v8", v8)):
        if np.asarray(x).dtype != np.uint8 or np.asarray(x).ndim != 4:
            raise TypeError(f"{name}: expected FP8 E4M3 codes as uint8 [B, H, T, d]")
    qd, kd, vd = (float(np.float32(s)) for s in (q_descale, k_descale, v_descale))
    q = e4m3_to_f64(q8) * qd
    k = e4m3_to_f64(k8) * kd
    v = e4m3_to_f64(v8) * vd
    return attention_fwd_f64(q, k, v, causal, scale, num_threads)


def attention_fwd_fp8_rows(q8, k8, v8, causal: bool, scale: float, q_descale: float, k_descale: float,
                           v_descale: float, rows):
    """``attention_fwd_fp8`` for selected rows only (numpy float64), for heads too long for the
    whole-head entry. ``rows`` holds ``(b, h, i)`` triples; returns ``(o, lse)`` with ``o``
    ``[len(rows), d]`` and ``lse`` ``[len(rows)]``. Each row is the same two-pass softmax over its
    visible keys (j <= i when causal) of the decoded, descaled values."""
    qd, kd, vd = (float(np.float32(s)) for s in (q_descale, k_descale, v_descale))
    d = np.asarray(q8).shape[-1]
    o, lse = np.empty((len(rows), d)), np.empty(len(rows))
    heads = {}
    for n, (b, h, i) in enumerate(rows):
        if (b, h) not in heads:
            heads[(b, h)] = (e4m3_to_f64(q8[b, h]) * qd, e4m3_to_f64(k8[b, h]) * kd,
                             e4m3_to_f64(v8[b, h]) * vd)
        q, k, v = heads[(b, h)]
        keys = i + 1 if causal else k.shape[0]
        s = scale * (k[:keys] @ q[i])
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        o[n] = (e @ v[:keys]) / l
        lse[n] = m + np.log(l)
    return o, lse

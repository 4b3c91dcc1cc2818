"""ctypes binding of libfa.so (include/fa.h): argument marshalling only.

Every step of the attention forward runs in the gfx950 HIP kernel behind ``fa_fwd``, and every step
of the backward in the kernels behind ``fa_bwd``; this module checks tensor metadata, allocates
outputs with torch when the caller gives none, and passes raw device pointers plus the current HIP
stream. There is no fallback: if ``libfa.so`` is missing or a call fails, it raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import re
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "fa.h")

FA_OK = 0
FA_ERR_NULL = -1
FA_ERR_INVALID_ARG = -2
FA_ERR_UNSUPPORTED_D = -3
FA_ERR_ALIGNMENT = -4
FA_ERR_HIP = -5
FA_ERR_TILE = -6
FA_ERR_SCRATCH = -7

_lib = None
_lib_lock = threading.Lock()


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"fa status {status}: {message}")
        self.status = status


class PlanInfo(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int), ("block_n", ctypes.c_int), ("waves", ctypes.c_int),
                ("q_blocks", ctypes.c_int), ("grid", ctypes.c_longlong),
                ("lds_bytes", ctypes.c_int), ("kv_tiles", ctypes.c_longlong), ("key_split", ctypes.c_int),
                ("head_group", ctypes.c_int)]


class _Int(ctypes.c_int):
    """A C ``int`` argument that refuses values outside its range (plain ctypes would wrap them
    silently, e.g. 2**32 + 5 to 5)."""

    @classmethod
    def from_param(cls, value):
        v = int(value)
        if not -(1 << 31) <= v < (1 << 31):
            raise OverflowError(f"{value} does not fit in a C int")
        return ctypes.c_int(v)


def lib():
    """Load libfa.so (once; safe from several threads). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lib_lock:
        if _lib is None:
            _lib = _load()
    return _lib


def _load():
    if not os.path.exists(LIB_PATH):
        raise FileNotFoundError(
            f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f = ctypes.c_void_p, _Int, ctypes.c_float
    L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    L.fa_fwd.restype = ctypes.c_int
    L.fa_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, i, i, i]
    L.fa_fwd_ex.restype = ctypes.c_int
    L.fa_fwd_plan.argtypes = [i, i, i, i, i, i, i, i, ctypes.POINTER(PlanInfo)]
    L.fa_fwd_plan.restype = ctypes.c_int
    L.fa_fwd_sparse.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, i, vp]
    L.fa_fwd_sparse.restype = ctypes.c_int
    L.fa_fwd_partial.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
    L.fa_fwd_partial.restype = ctypes.c_int
    L.fa_merge.argtypes = [vp, vp, i, vp, vp, i, i, i, i, vp]
    L.fa_merge.restype = ctypes.c_int
    L.fa_splitkv_workspace_bytes.argtypes = [i, i, i, i, i]
    L.fa_splitkv_workspace_bytes.restype = ctypes.c_size_t
    L.fa_splitkv_splits.argtypes = [i, i, i, i, i]
    L.fa_splitkv_splits.restype = ctypes.c_int
    L.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, ctypes.c_size_t, vp]
    L.fa_fwd_splitkv.restype = ctypes.c_int
    L.fa_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    L.fa_fwd_splitkv_noalloc.restype = ctypes.c_int
    L.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, f, f, f, vp]
    L.fa_fwd_fp8.restype = ctypes.c_int
    L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    L.fa_bwd.restype = ctypes.c_int
    L.fa_strerror.argtypes = [i]
    L.fa_strerror.restype = ctypes.c_char_p
    return L


def header_functions():
    """Names of the functions include/fa.h declares."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"^(?:int|size_t|const char\*)\s+(fa_\w+)\s*\(", text, flags=re.M)))


def strerror(status: int) -> str:
    return lib().fa_strerror(int(status)).decode()


def _check(status: int):
    if status != FA_OK:
        raise FaError(status, strerror(status))


def plan(B: int, H: int, T: int, d: int, causal: bool = True, block_m: int = 0, block_n: int = 0,
         waves: int = 0) -> dict:
    """Launch plan (tile shape, grid, LDS bytes, K/V tiles) that fa_fwd / fa_fwd_ex would use."""
    info = PlanInfo()
    _check(lib().fa_fwd_plan(B, H, T, d, int(bool(causal)), block_m, block_n, waves, ctypes.byref(info)))
    return {name: getattr(info, name) for name, _ in PlanInfo._fields_}


def _check_inputs(q, k, v, *more, keys_may_differ=False):
    """Dtype, device, rank and contiguity of q, k, v (and of ``more``, shaped like q). With
    ``keys_may_differ`` k and v may hold another number of keys than q has queries."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), *more):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, T, d], got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    same = (q.shape == k.shape == v.shape) if not keys_may_differ else (
        k.shape == v.shape and q.shape[:2] == k.shape[:2] and q.shape[3] == k.shape[3])
    if not same:
        raise ValueError(f"q, k, v shapes do not fit: {tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")
    for name, t in more:
        if t.shape != q.shape or t.device != q.device:
            raise ValueError(f"{name} must be shaped like q and on q's device")


def _outputs(q, out, lse):
    import torch

    B, H, T, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    elif (out.dtype != torch.bfloat16 or out.shape != q.shape or not out.is_contiguous()
          or out.device != q.device):
        raise ValueError("out must be a contiguous bfloat16 tensor shaped like q on q's device")
    if lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    elif (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, T) or not lse.is_contiguous()
          or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 tensor [B, H, T] on q's device")
    return out, lse


def _stream_handle(device, stream):
    import torch

    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def fwd(q, k, v, causal: bool = True, scale: float | None = None, out=None, lse=None, stream=None):
    """Exact attention forward on the GPU: returns ``(o, lse)``.

    q, k, v: contiguous bfloat16 ``[B, H, T, d]`` GPU tensors (d = 64 or 128). ``o`` is bfloat16
    like q; ``lse`` is float32 ``[B, H, T]`` (natural log). ``scale`` defaults to 1/sqrt(d).
    Launches on ``stream`` (a torch stream; default: the current stream of q's device).
    """
    import torch

    _check_inputs(q, k, v)
    out, lse = _outputs(q, out, lse)
    B, H, T, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        _check(lib().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                            B, H, T, d, int(bool(causal)), scale, _stream_handle(q.device, stream)))
    return out, lse


def fwd_ex(q, k, v, block_m: int, block_n: int, waves: int, causal: bool = True,
           scale: float | None = None, out=None, lse=None, stream=None):
    """``fwd`` with the tile shape forced (``fa_fwd_ex``), for the tile-shape study."""
    import torch

    _check_inputs(q, k, v)
    out, lse = _outputs(q, out, lse)
    B, H, T, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        _check(lib().fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                               lse.data_ptr(), B, H, T, d, int(bool(causal)), scale,
                               _stream_handle(q.device, stream), block_m, block_n, waves))
    return out, lse


def fwd_fp8(q8, k8, v8, q_descale: float, k_descale: float, v_descale: float, causal: bool = True,
            scale: float | None = None, out=None, lse=None, stream=None):
    """Attention forward on FP8 E4M3 inputs (``fa_fwd_fp8``): returns bf16 ``o`` and float32 ``lse``.

    ``q8``, ``k8``, ``v8``: contiguous ``[B, H, T, d]`` GPU tensors of E4M3 codes (``torch.uint8`` or
    ``torch.float8_e4m3fn``) standing for ``code * descale`` with one descale factor per tensor.
    ``scale`` defaults to 1/sqrt(d).
    """
    import torch

    for name, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        if not isinstance(t, torch.Tensor) or t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError(f"{name} must be a uint8 or float8_e4m3fn torch.Tensor")
        if not t.is_cuda or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, T, d] GPU tensor")
        if t.shape != q8.shape or t.device != q8.device:
            raise ValueError("q8, k8, v8 must have one shape and one device")
    B, H, T, d = q8.shape
    if out is None:
        out = torch.empty((B, H, T, d), dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=q8.device)
    if (out.dtype != torch.bfloat16 or tuple(out.shape) != (B, H, T, d) or not out.is_contiguous()
            or out.device != q8.device):
        raise ValueError("out must be a contiguous bfloat16 tensor [B, H, T, d] on q8's device")
    if (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, T) or not lse.is_contiguous()
            or lse.device != q8.device):
        raise ValueError("lse must be a contiguous float32 tensor [B, H, T] on q8's device")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with torch.cuda.device(q8.device):
        _check(lib().fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(),
                                lse.data_ptr(), B, H, T, d, int(bool(causal)), scale, float(q_descale),
                                float(k_descale), float(v_descale), _stream_handle(q8.device, stream)))
    return out, lse


def _like(q, t, name, dtype=None, shape=None):
    import torch

    dtype = q.dtype if dtype is None else dtype
    shape = tuple(q.shape) if shape is None else shape
    if t is None:
        return torch.empty(shape, dtype=dtype, device=q.device)
    if t.dtype != dtype or tuple(t.shape) != shape or not t.is_contiguous() or t.device != q.device:
        raise ValueError(f"{name} must be a contiguous {dtype} tensor {shape} on q's device")
    return t


def bwd(q, k, v, o, lse, dout, causal: bool = True, scale: float | None = None, dq=None, dk=None,
        dv=None, delta=None, stream=None):
    """Exact attention backward on the GPU (``fa_bwd``): returns ``(dq, dk, dv, delta)``.

    ``o`` and ``lse`` are the outputs of ``fwd`` for the same q, k, v, causal and scale; ``dout`` is
    the gradient of the loss with respect to ``o``. All bfloat16 tensors are contiguous
    ``[B, H, T, d]`` on the GPU (d = 64 or 128); lse is float32 ``[B, H, T]``. Returns bfloat16 gradients shaped
    like q and ``delta`` float32 ``[B, H, T]`` (``dO_i . O_i``).
    """
    import torch

    _check_inputs(q, k, v, ("o", o), ("dout", dout))
    B, H, T, d = q.shape
    if (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, T) or not lse.is_contiguous()
            or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 tensor [B, H, T] on q's device")
    dq, dk, dv = _like(q, dq, "dq"), _like(q, dk, "dk"), _like(q, dv, "dv")
    delta = _like(q, delta, "delta", torch.float32, (B, H, T))
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        _check(lib().fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                            delta.data_ptr(), B, H, T, d, int(bool(causal)), scale,
                            _stream_handle(q.device, stream)))
    return dq, dk, dv, delta


SPARSE_BLOCK_M = 128  # FA_SPARSE_BLOCK_M: query rows per mask block
SPARSE_BLOCK_N = 64   # FA_SPARSE_BLOCK_N: keys per mask block


def sparse_mask_shape(T: int, mask_heads: int = 1):
    """Shape of the block mask ``fwd_sparse`` takes for sequence length T."""
    return (mask_heads, -(-T // SPARSE_BLOCK_M), -(-T // SPARSE_BLOCK_N))


def fwd_sparse(q, k, v, block_mask, causal: bool = True, scale: float | None = None, out=None,
               lse=None, stream=None):
    """Block-sparse attention forward (``fa_fwd_sparse``): returns ``(o, lse)``.

    ``block_mask`` is a contiguous uint8 GPU tensor ``[mask_heads, ceil(T/128), ceil(T/64)]`` with
    ``mask_heads`` 1 or B*H; nonzero blocks are computed, the others skipped. Rows with no visible
    key get o = 0 and lse = -inf.
    """
    import torch

    _check_inputs(q, k, v)
    out, lse = _outputs(q, out, lse)
    B, H, T, d = q.shape
    if (not isinstance(block_mask, torch.Tensor) or block_mask.dtype != torch.uint8
            or not block_mask.is_contiguous() or block_mask.device != q.device):
        raise TypeError("block_mask must be a contiguous uint8 tensor on q's device")
    mh = block_mask.shape[0] if block_mask.dim() == 3 else -1
    if mh not in (1, B * H) or tuple(block_mask.shape) != sparse_mask_shape(T, mh):
        raise ValueError(f"block_mask must be {sparse_mask_shape(T, 1)} or {sparse_mask_shape(T, B * H)}")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        _check(lib().fa_fwd_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr(), B, H, T, d, int(bool(causal)), scale,
                                   block_mask.data_ptr(), mh, _stream_handle(q.device, stream)))
    return out, lse


PARTIAL_KEY_ALIGN = 64  # FA_PARTIAL_KEY_ALIGN


def fwd_partial(q, k, v, k_begin: int, k_end: int, causal: bool = True, scale: float | None = None,
                o_part=None, lse_part=None, stream=None):
    """Attention over the keys [k_begin, k_end) only (``fa_fwd_partial``): ``(o_part, lse_part)``.

    q is ``[B, H, T, d]``, k and v ``[B, H, Tk, d]`` (Tk may differ from T; with the causal mask
    the queries are the last T positions of the keys' sequence). ``o_part`` is float32
    ``[B, H, T, d]`` (normalised over the range) and ``lse_part`` float32 ``[B, H, T]``; rows with
    no visible key in the range get 0 and -inf. k_begin must be a multiple of 64 and k_end a
    multiple of 64 or Tk.
    """
    import torch

    _check_inputs(q, k, v, keys_may_differ=True)
    B, H, T, d = q.shape
    Tk = k.shape[2]
    o_part = _like(q, o_part, "o_part", torch.float32)
    lse_part = _like(q, lse_part, "lse_part", torch.float32, (B, H, T))
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        _check(lib().fa_fwd_partial(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_part.data_ptr(),
                                    lse_part.data_ptr(), B, H, T, Tk, d, int(bool(causal)), scale,
                                    int(k_begin), int(k_end), _stream_handle(q.device, stream)))
    return o_part, lse_part


def splitkv_splits(B: int, H: int, T: int, Tk: int, d: int) -> int:
    """The split count ``fa_splitkv_splits`` suggests for this shape (enough workgroups to fill
    the GPU, ranges of at least 512 keys)."""
    return int(lib().fa_splitkv_splits(B, H, T, Tk, d))


def splitkv_workspace_bytes(B: int, H: int, T: int, d: int, n_splits: int) -> int:
    return int(lib().fa_splitkv_workspace_bytes(B, H, T, d, n_splits))


def fwd_splitkv(q, k, v, causal: bool = True, scale: float | None = None, n_splits: int | None = None,
                out=None, lse=None, workspace=None, stream=None):
    """Attention with the keys split into ranges that run side by side, then merged
    (``fa_fwd_splitkv``): returns bf16 ``o`` ``[B, H, T, d]`` and float32 ``lse``.

    For few queries against many keys (T << Tk). ``n_splits`` defaults to ``splitkv_splits``;
    ``workspace`` (a uint8 GPU tensor of at least ``splitkv_workspace_bytes`` bytes) is allocated
    with torch when not given.
    """
    import torch

    _check_inputs(q, k, v, keys_may_differ=True)
    B, H, T, d = q.shape
    Tk = k.shape[2]
    out, lse = _outputs(q, out, lse)
    n_splits = splitkv_splits(B, H, T, Tk, d) if n_splits is None else int(n_splits)
    need = splitkv_workspace_bytes(B, H, T, d, n_splits) if n_splits >= 1 else 0
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if workspace.dtype != torch.uint8 or workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on q's device")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        _check(lib().fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                    lse.data_ptr(), B, H, T, Tk, d, int(bool(causal)), scale, n_splits,
                                    workspace.data_ptr(), workspace.numel(),
                                    _stream_handle(q.device, stream)))
    return out, lse


def fwd_splitkv_noalloc(q, k, v, causal: bool = True, scale: float | None = None,
                        n_splits: int | None = None, out=None, lse=None, stream=None):
    """``fa_fwd_splitkv_noalloc``: split-KV attention whose partial results go through the library's
    fixed device buffer (no workspace, no allocation by the library). Returns bf16 ``o`` and float32
    ``lse``; pass ``out`` and ``lse`` to keep this call free of allocations too.
    """
    import torch

    _check_inputs(q, k, v, keys_may_differ=True)
    B, H, T, d = q.shape
    Tk = k.shape[2]
    out, lse = _outputs(q, out, lse)
    n_splits = splitkv_splits(B, H, T, Tk, d) if n_splits is None else int(n_splits)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        _check(lib().fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                            lse.data_ptr(), B, H, T, Tk, d, int(bool(causal)), scale,
                                            n_splits, _stream_handle(q.device, stream)))
    return out, lse


def merge(o_parts, lse_parts, out=None, lse=None, stream=None):
    """Log-space merge of partial results (``fa_merge``): returns bf16 ``o`` and float32 ``lse``.

    ``o_parts`` float32 ``[n, B, H, T, d]``, ``lse_parts`` float32 ``[n, B, H, T]`` (contiguous,
    on the GPU), e.g. stacked ``fwd_partial`` outputs over disjoint key ranges.
    """
    import torch

    if (o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32 or o_parts.dim() != 5
            or tuple(lse_parts.shape) != tuple(o_parts.shape[:4]) or not o_parts.is_contiguous()
            or not lse_parts.is_contiguous() or not o_parts.is_cuda or lse_parts.device != o_parts.device):
        raise ValueError("o_parts must be float32 [n, B, H, T, d] and lse_parts float32 [n, B, H, T], "
                         "contiguous, on one GPU")
    n, B, H, T, d = o_parts.shape
    if out is None:
        out = torch.empty((B, H, T, d), dtype=torch.bfloat16, device=o_parts.device)
    if lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=o_parts.device)
    if (out.dtype != torch.bfloat16 or tuple(out.shape) != (B, H, T, d) or not out.is_contiguous()
            or out.device != o_parts.device):
        raise ValueError("out must be a contiguous bfloat16 tensor [B, H, T, d] on the parts' device")
    if (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, T) or not lse.is_contiguous()
            or lse.device != o_parts.device):
        raise ValueError("lse must be a contiguous float32 tensor [B, H, T] on the parts' device")
    with torch.cuda.device(o_parts.device):
        _check(lib().fa_merge(o_parts.data_ptr(), lse_parts.data_ptr(), n, out.data_ptr(),
                              lse.data_ptr(), B, H, T, d, _stream_handle(o_parts.device, stream)))
    return out, lse

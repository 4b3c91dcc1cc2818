"""MI355X-native exact tiled attention: forward (dense, block-sparse, key ranges with a log-space
merge, FP8 inputs) and its backward.

The work runs in hand-written gfx950 HIP kernels behind the C-ABI library ``libfa.so``
(``include/fa.h``); this package is its thin Python binding. PyTorch provides device memory and
streams only.
"""
from .fa import (FaError, bwd, fwd, fwd_ex, fwd_fp8, fwd_partial, fwd_sparse, fwd_splitkv,
                 fwd_splitkv_noalloc, merge, plan, sparse_mask_shape, splitkv_splits,
                 splitkv_workspace_bytes, strerror)

__all__ = ["FaError", "bwd", "fwd", "fwd_ex", "fwd_fp8", "fwd_partial", "fwd_sparse", "fwd_splitkv",
           "fwd_splitkv_noalloc", "merge", "plan", "sparse_mask_shape", "splitkv_splits",
           "splitkv_workspace_bytes", "strerror"]

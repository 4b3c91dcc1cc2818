"""MI355X-native exact tiled attention: forward, and its backward by recomputation.

The work runs in hand-written gfx950 HIP kernels behind the C-ABI library ``libfa.so``
(``include/fa.h``); this package is its thin Python binding. PyTorch provides device memory and
streams only.
"""
from .fa import FaError, bwd, fwd, fwd_ex, plan, strerror

__all__ = ["FaError", "bwd", "fwd", "fwd_ex", "plan", "strerror"]

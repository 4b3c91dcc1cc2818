"""MI355X-native exact tiled attention forward.

The work runs in a hand-written gfx950 HIP kernel behind the C-ABI library ``libfa.so``
(``include/fa.h``); this package is its thin Python binding. PyTorch provides device memory and
streams only.
"""
from .fa import FaError, fwd, fwd_ex, plan, strerror

__all__ = ["FaError", "fwd", "fwd_ex", "plan", "strerror"]

"""Fused exact attention for AMD Instinct MI355X (gfx950).

The compute lives in libfa.so (HIP kernels behind a C ABI, include/fa.h);
this package is its thin Python binding.
"""

from .attention import (FaArgError, bwd, flash_attn_func, flash_attn_qkvpacked_func, fwd,
                        fwd_fp8, merge, workspace_bytes)
from .mha import FlashMHA

__all__ = ["fwd", "fwd_fp8", "bwd", "merge", "flash_attn_func", "flash_attn_qkvpacked_func",
           "workspace_bytes", "FlashMHA", "FaArgError"]

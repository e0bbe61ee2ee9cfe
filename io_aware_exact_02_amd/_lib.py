"""ctypes view of libfa.so (the C ABI in include/fa.h).

Argument marshalling only: this module turns Python values into the C
types of the ABI.  It raises if the library is missing -- there is no
fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")
# The same library built with LDS poisoning (FA_POISON_LDS=1), for tests.
POISON_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_poison.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP, FA_ERR_TOO_LARGE = 0, 1, 2, 3, 4
FA_F16, FA_BF16 = 0, 1

# Every symbol include/fa.h declares.
EXPORTS = ("fa_fwd", "fa_fwd_qk", "fa_fwd_split", "fa_fwd_split_workspace_bytes",
           "fa_fwd_split_count", "fa_fwd_fp8", "fa_bwd", "fa_bwd_stages", "fa_bwd_qk",
           "fa_bwd_workspace_bytes", "fa_bwd_qk_workspace_bytes",
           "fa_bwd_qk_workspace_bytes_for", "fa_bwd_noalloc",
           "fa_bwd_noalloc_max_bytes", "fa_merge", "fa_status_str", "fa_version")
STAGE_PREPROCESS, STAGE_DKDV, STAGE_DQ, STAGE_ALL = 1, 2, 4, 7


class Stride3(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("n", ctypes.c_int64), ("h", ctypes.c_int64)]


class FwdStrides(ctypes.Structure):
    _fields_ = [(n, Stride3) for n in ("q", "k", "v", "o")]


class BwdStrides(ctypes.Structure):
    _fields_ = [(n, Stride3) for n in ("q", "k", "v", "o", "dout", "dq", "dk", "dv")]


class FaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libfa.so once; raise ImportError if it has not been built."""
    global _lib
    if _lib is None:
        _lib = open_library(LIB_PATH)
    return _lib


def open_library(path: str) -> ctypes.CDLL:
    """Load a build of the library at ``path`` and declare its signatures."""
    if not os.path.exists(path):
        raise ImportError(
            f"{path} not found: build the HIP library first "
            "(python -m io_aware_exact_02_amd.build)")
    lib = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i,
                           ctypes.POINTER(FwdStrides), vp]
    lib.fa_fwd.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i,
                           ctypes.POINTER(BwdStrides), vp, ctypes.c_size_t, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_stages.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i,
                                  ctypes.POINTER(BwdStrides), vp, ctypes.c_size_t,
                                  ctypes.c_uint, vp]
    lib.fa_bwd_stages.restype = i
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_fwd_qk.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i,
                              ctypes.POINTER(FwdStrides), vp]
    lib.fa_fwd_qk.restype = i
    lib.fa_fwd_split.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i,
                                 ctypes.POINTER(FwdStrides), i, vp, ctypes.c_size_t, vp]
    lib.fa_fwd_split.restype = i
    lib.fa_fwd_split_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_fwd_split_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_fwd_split_count.argtypes = [i, i, i, i, i, i]
    lib.fa_fwd_split_count.restype = i
    lib.fa_bwd_qk.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i,
                              ctypes.POINTER(BwdStrides), vp, ctypes.c_size_t, ctypes.c_uint, vp]
    lib.fa_bwd_qk.restype = i
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i,
                                   ctypes.POINTER(BwdStrides), vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_bwd_noalloc_max_bytes.argtypes = []
    lib.fa_bwd_noalloc_max_bytes.restype = ctypes.c_size_t
    lib.fa_bwd_qk_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_bwd_qk_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd_qk_workspace_bytes_for.argtypes = [i, i, i, i, i, i]
    lib.fa_bwd_qk_workspace_bytes_for.restype = ctypes.c_size_t
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i,
                               ctypes.POINTER(FwdStrides), vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_merge.argtypes = [vp, vp, i, vp, vp, i, i, i, i, i, vp]
    lib.fa_merge.restype = i
    lib.fa_status_str.argtypes = [i]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = ctypes.c_char_p
    return lib


def check(status: int, what: str) -> None:
    if status != FA_OK:
        msg = load().fa_status_str(status).decode()
        if status == FA_ERR_HIP:
            raise FaError(status, f"{what}: {msg}")
        raise FaError(status, f"{what}: {msg}")

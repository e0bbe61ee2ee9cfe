"""CPU-side checks of the C ABI and the Python binding (no GPU needed).

The library must load, export every function include/fa.h declares, and
reject invalid arguments before making any HIP call.  Only argument-error
paths are exercised here; nothing is launched.
"""

import ctypes
import os
import re

import pytest
import torch

from io_aware_exact_02_amd import _lib
from io_aware_exact_02_amd import attention as fa

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "fa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libfa.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(fa_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    lib = _lib.load()
    declared = _declared_functions()
    assert set(declared) == set(_lib.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    lib = _lib.load()
    assert lib.fa_version().decode().startswith("fa-gfx950")
    for st in range(5):
        assert lib.fa_status_str(st)
    assert b"unknown" in lib.fa_status_str(99)


def test_workspace_bytes_is_linear_in_n():
    lib = _lib.load()

    def a256(x):
        return (x + 255) // 256 * 256

    # Dvec, the int32 dQ accumulator, three maxima per 16-row block, one
    # fixed-point bound per head, and -- for launches with fewer than 512 key
    # blocks (256 keys), whose query range a causal mask splits into
    # S = min(8, ceil(512 / blocks), query tiles) segments (tiles of 64 rows
    # at head_dim 64, 32 at head_dim 128) -- S fp32 partial dK and dV sums:
    # O(N*D) per head, no N*N term.
    def want_bytes(B, H, N, D):
        heads, rows = B * H, B * H * N
        bkv, bq = 256, (64 if D == 64 else 32)
        blocks = heads * ((N + bkv - 1) // bkv)
        segs = min(8, -(-512 // blocks), -(-N // bq)) if blocks < 512 else 1
        part = 2 * a256(4 * segs * heads * N * D) if segs > 1 else 0
        return (a256(4 * rows) + a256(4 * rows * D)
                + a256(4 * 3 * heads * ((N + 15) // 16)) + a256(4 * heads) + part)

    for (B, H, N, D) in [(1, 1, 1, 64), (2, 12, 2048, 64), (1, 16, 16384, 64), (1, 8, 8192, 128),
                         (3, 5, 1000, 128), (1, 2, 16384, 64)]:
        want = want_bytes(B, H, N, D)
        assert lib.fa_bwd_workspace_bytes(B, H, N, D) == want
        assert lib.fa_bwd_workspace_bytes(B, H, 2 * N, D) <= want_bytes(B, H, 2 * N, D)
        assert want_bytes(B, H, 2 * N, D) < 2 * want + 6 * 256
    assert lib.fa_bwd_workspace_bytes(0, 1, 1, 64) == 0


# Fake device pointers: never dereferenced because validation fails first.
P = 0x10000
ARGS_OK = dict(B=1, H=1, N=128, D=64, causal=0, scale=0.125, dtype=_lib.FA_BF16)


def _fwd(q=P, k=P, v=P, o=P, lse=P, strides=None, **kw):
    a = dict(ARGS_OK, **kw)
    st = ctypes.byref(strides) if strides is not None else None
    return _lib.load().fa_fwd(q, k, v, o, lse, a["B"], a["H"], a["N"], a["D"], a["causal"],
                              a["scale"], a["dtype"], st, None)


def _bwd(ptrs=None, ws=P, ws_bytes=1 << 40, strides=None, **kw):
    a = dict(ARGS_OK, **kw)
    p = [P] * 9 if ptrs is None else ptrs
    st = ctypes.byref(strides) if strides is not None else None
    return _lib.load().fa_bwd(*p, a["B"], a["H"], a["N"], a["D"], a["causal"], a["scale"],
                              a["dtype"], st, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), _lib.FA_ERR_INVALID_ARG),
    (dict(lse=None), _lib.FA_ERR_INVALID_ARG),
    (dict(B=0), _lib.FA_ERR_INVALID_ARG),
    (dict(H=-1), _lib.FA_ERR_INVALID_ARG),
    (dict(N=0), _lib.FA_ERR_INVALID_ARG),
    (dict(causal=2), _lib.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _lib.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), _lib.FA_ERR_INVALID_ARG),
    (dict(dtype=7), _lib.FA_ERR_INVALID_ARG),
    (dict(D=32), _lib.FA_ERR_UNSUPPORTED),
    (dict(D=96), _lib.FA_ERR_UNSUPPORTED),
    (dict(D=256), _lib.FA_ERR_UNSUPPORTED),
    (dict(q=P + 8), _lib.FA_ERR_UNSUPPORTED),
    (dict(o=P + 2), _lib.FA_ERR_UNSUPPORTED),
    (dict(lse=P + 2), _lib.FA_ERR_UNSUPPORTED),
    (dict(B=1 << 16, H=1 << 12, N=1 << 12), _lib.FA_ERR_UNSUPPORTED),
])
def test_fwd_rejects_before_launch(kw, expect):
    assert _fwd(**kw) == expect


def test_fwd_rejects_bad_strides():
    good = _lib.Stride3(128 * 64, 64, 64)
    for bad in (_lib.Stride3(128 * 64, 60, 64), _lib.Stride3(-8, 64, 64),
                _lib.Stride3(128 * 64, 64, 4)):
        for field in ("q", "k", "v", "o"):
            s = _lib.FwdStrides(good, good, good, good)
            setattr(s, field, bad)
            assert _fwd(strides=s) == _lib.FA_ERR_UNSUPPORTED, (field, bad.n, bad.h)


def test_bwd_rejects_before_launch():
    lib = _lib.load()
    need = lib.fa_bwd_workspace_bytes(1, 1, 128, 64)   # the causal size
    assert _bwd(ws_bytes=need - 1, causal=1) == _lib.FA_ERR_INVALID_ARG
    need_nc = lib.fa_bwd_qk_workspace_bytes_for(1, 1, 128, 128, 64, 0)
    assert need_nc <= need
    assert _bwd(ws_bytes=need_nc - 1) == _lib.FA_ERR_INVALID_ARG
    assert _bwd(ws=None) == _lib.FA_ERR_INVALID_ARG
    assert _bwd(ws=P + 16) == _lib.FA_ERR_UNSUPPORTED       # workspace needs 256 B alignment
    for i in range(9):
        ptrs = [P] * 9
        ptrs[i] = None
        assert _bwd(ptrs=ptrs) == _lib.FA_ERR_INVALID_ARG, i
    ptrs = [P] * 9
    ptrs[6] = P + 4                                           # dq misaligned
    assert _bwd(ptrs=ptrs) == _lib.FA_ERR_UNSUPPORTED
    assert _bwd(D=80) == _lib.FA_ERR_UNSUPPORTED
    assert _bwd(causal=-1) == _lib.FA_ERR_INVALID_ARG
    good = _lib.Stride3(128 * 64, 64, 64)
    s = _lib.BwdStrides(*([good] * 8))
    s.dk = _lib.Stride3(128 * 64, 68, 64)
    assert _bwd(strides=s) == _lib.FA_ERR_UNSUPPORTED


def test_bwd_stages_rejects_bad_mask():
    lib = _lib.load()
    for stages in (0, 8, 15, 0xFFFFFFFF):
        assert lib.fa_bwd_stages(*([P] * 9), 1, 1, 128, 64, 0, 0.125, _lib.FA_BF16, None, P,
                                 1 << 40, stages, None) == _lib.FA_ERR_INVALID_ARG


def test_python_binding_rejects_bad_inputs_without_gpu():
    q = torch.zeros(1, 16, 2, 64, dtype=torch.float32)
    with pytest.raises(fa.FaArgError, match="float16 / bfloat16"):
        fa.fwd(q, q, q)
    qb = q.to(torch.bfloat16)
    with pytest.raises(fa.FaArgError, match="GPU"):
        fa.fwd(qb, qb, qb)
    with pytest.raises(fa.FaArgError, match="head_dim"):
        x = torch.zeros(1, 16, 2, 32, dtype=torch.bfloat16)
        fa._check_inputs(x, x, x)
    with pytest.raises(fa.FaArgError, match=r"\[B, N, 3, H, D\]"):
        fa.flash_attn_qkvpacked_func(torch.zeros(1, 16, 2, 2, 64, dtype=torch.float16))


def test_unequal_length_entry_points_reject_before_launch():
    lib = _lib.load()

    def fwd_qk(Nq=128, Nk=256, **kw):
        a = dict(ARGS_OK, **kw)
        return lib.fa_fwd_qk(P, P, P, P, P, a["B"], a["H"], Nq, Nk, a["D"], a["causal"],
                             a["scale"], a["dtype"], None, None)

    assert fwd_qk(Nq=0) == _lib.FA_ERR_INVALID_ARG
    assert fwd_qk(Nk=0) == _lib.FA_ERR_INVALID_ARG
    assert fwd_qk(Nk=-5) == _lib.FA_ERR_INVALID_ARG
    assert fwd_qk(D=48) == _lib.FA_ERR_UNSUPPORTED
    assert fwd_qk(causal=3) == _lib.FA_ERR_INVALID_ARG
    # strides are checked against each tensor's own length
    good_q, good_k = _lib.Stride3(128 * 64, 64, 64), _lib.Stride3(256 * 64, 64, 64)
    s = _lib.FwdStrides(good_q, good_k, good_k, good_q)
    s.k = _lib.Stride3(256 * 64, 66, 64)
    assert lib.fa_fwd_qk(P, P, P, P, P, 1, 1, 128, 256, 64, 0, 0.125, _lib.FA_BF16,
                         ctypes.byref(s), None) == _lib.FA_ERR_UNSUPPORTED

    need = lib.fa_bwd_qk_workspace_bytes(1, 1, 128, 256, 64)
    a256 = lambda x: (x + 255) // 256 * 256
    # one key block: the partial dK, dV sums of two query segments over Nk keys
    assert need == (a256(4 * 128) + a256(4 * 128 * 64) + a256(4 * 3 * (256 // 16))
                    + a256(4) + 2 * a256(4 * 2 * 256 * 64))
    assert lib.fa_bwd_qk_workspace_bytes(1, 1, 0, 256, 64) == 0
    assert lib.fa_bwd_qk_workspace_bytes(1, 1, 5, 5, 64) == lib.fa_bwd_workspace_bytes(1, 1, 5, 64)

    def bwd_qk(ws_bytes=1 << 40, stages=_lib.STAGE_ALL, Nq=128, Nk=256, **kw):
        a = dict(ARGS_OK, **kw)
        return lib.fa_bwd_qk(*([P] * 9), a["B"], a["H"], Nq, Nk, a["D"], a["causal"],
                             a["scale"], a["dtype"], None, P, ws_bytes, stages, None)

    assert bwd_qk(ws_bytes=need - 1, causal=1) == _lib.FA_ERR_INVALID_ARG
    # One key block: a non-causal launch splits its two query tiles too.
    assert lib.fa_bwd_qk_workspace_bytes_for(1, 1, 128, 256, 64, 0) == need
    assert lib.fa_bwd_qk_workspace_bytes_for(1, 1, 128, 256, 64, 1) == need
    # 192 key blocks (B2 H12 N2048 D64): a non-causal launch runs one query
    # segment, so its workspace has no partial sums; a causal one runs three.
    # The causal size serves either mask.
    nc = lib.fa_bwd_qk_workspace_bytes_for(2, 12, 2048, 2048, 64, 0)
    c = lib.fa_bwd_qk_workspace_bytes_for(2, 12, 2048, 2048, 64, 1)
    assert c == lib.fa_bwd_workspace_bytes(2, 12, 2048, 64)
    assert c - nc == 2 * a256(4 * 3 * 24 * 2048 * 64)
    assert bwd_qk(ws_bytes=nc - 1, causal=0, B=2, H=12, Nq=2048, Nk=2048) == _lib.FA_ERR_INVALID_ARG
    assert lib.fa_bwd_qk_workspace_bytes_for(1, 1, 128, 256, 64, 2) == 0
    assert lib.fa_bwd_qk_workspace_bytes_for(1, 1, 0, 256, 64, 0) == 0
    assert bwd_qk(Nk=0) == _lib.FA_ERR_INVALID_ARG
    assert bwd_qk(stages=0) == _lib.FA_ERR_INVALID_ARG
    assert bwd_qk(stages=16) == _lib.FA_ERR_INVALID_ARG
    # one head's dQ accumulator must stay below 2^31 bytes
    assert bwd_qk(Nq=1 << 23, Nk=8, D=64) == _lib.FA_ERR_UNSUPPORTED


def test_merge_rejects_before_launch():
    lib = _lib.load()

    def merge(o_parts=P, lse_parts=P, n=3, o=P, lse=P, B=1, H=2, N=64, D=64,
              dtype=_lib.FA_BF16):
        return lib.fa_merge(o_parts, lse_parts, n, o, lse, B, H, N, D, dtype, None)

    assert merge(n=0) == _lib.FA_ERR_INVALID_ARG
    assert merge(o_parts=None) == _lib.FA_ERR_INVALID_ARG
    assert merge(lse=None) == _lib.FA_ERR_INVALID_ARG
    assert merge(N=0) == _lib.FA_ERR_INVALID_ARG
    assert merge(dtype=5) == _lib.FA_ERR_INVALID_ARG
    assert merge(D=100) == _lib.FA_ERR_UNSUPPORTED
    assert merge(o=P + 8) == _lib.FA_ERR_UNSUPPORTED
    assert merge(lse_parts=P + 2) == _lib.FA_ERR_UNSUPPORTED


def test_python_binding_checks_unequal_lengths_without_gpu():
    q = torch.zeros(1, 16, 2, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 40, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(fa.FaArgError, match="GPU"):
        fa.fwd(q, k, k)                       # lengths accepted, device rejected
    with pytest.raises(fa.FaArgError, match="differ"):
        fa.fwd(q, torch.zeros(1, 40, 3, 64, dtype=torch.bfloat16),
               torch.zeros(1, 40, 3, 64, dtype=torch.bfloat16))
    with pytest.raises(fa.FaArgError, match="shape mismatch"):
        fa.fwd(q, k, torch.zeros(1, 41, 2, 64, dtype=torch.bfloat16))
    with pytest.raises(fa.FaArgError, match="lse_parts"):
        fa.merge(torch.zeros(2, 1, 16, 2, 64, dtype=torch.bfloat16),
                 torch.zeros(2, 1, 2, 17, dtype=torch.float32))


def test_huge_n_stride_rejected():
    """Tiles are addressed with 32-bit element offsets: n strides of 2^24
    elements or more are refused before any launch, in every entry point."""
    lib = _lib.load()
    s = _lib.Stride3(64 * 2 * 64, 2 * 64, 64)
    huge = _lib.Stride3(1 << 30, 1 << 24, 64)
    fst = _lib.FwdStrides(s, huge, s, s)
    assert lib.fa_fwd(P, P, P, P, P, 1, 2, 64, 64, 0, 0.125, _lib.FA_BF16,
                      ctypes.byref(fst), None) == _lib.FA_ERR_UNSUPPORTED
    bst = _lib.BwdStrides(s, s, s, s, s, s, s, huge)
    assert lib.fa_bwd(P, P, P, P, P, P, P, P, P, 1, 2, 64, 64, 0, 0.125, _lib.FA_BF16,
                      ctypes.byref(bst), P, 1 << 30, None) == _lib.FA_ERR_UNSUPPORTED


def test_fp8_rejects_before_launch():
    lib = _lib.load()

    def f8(q=P, k=P, v=P, o=P, lse=P, dq=None, dk=None, dv=None, B=1, H=2, Nq=64, Nk=64,
           D=64, causal=0, scale=0.125, out=_lib.FA_BF16, strides=None):
        st = None if strides is None else ctypes.byref(strides)
        return lib.fa_fwd_fp8(q, k, v, o, lse, dq, dk, dv, B, H, Nq, Nk, D, causal, scale, out,
                              st, None)

    assert f8(q=None) == _lib.FA_ERR_INVALID_ARG
    assert f8(lse=None) == _lib.FA_ERR_INVALID_ARG
    assert f8(Nk=0) == _lib.FA_ERR_INVALID_ARG
    assert f8(out=7) == _lib.FA_ERR_INVALID_ARG
    assert f8(causal=2) == _lib.FA_ERR_INVALID_ARG
    assert f8(scale=float("nan")) == _lib.FA_ERR_INVALID_ARG
    assert f8(D=96) == _lib.FA_ERR_UNSUPPORTED
    assert f8(v=P + 8) == _lib.FA_ERR_UNSUPPORTED
    assert f8(dk=P + 2) == _lib.FA_ERR_UNSUPPORTED
    s = _lib.Stride3(64 * 2 * 64, 2 * 64, 64)
    ok = _lib.FwdStrides(s, s, s, s)
    bad8 = _lib.FwdStrides(_lib.Stride3(64 * 2 * 64, 2 * 64 + 8, 64), s, s, s)  # 8, not 16
    huge = _lib.FwdStrides(s, _lib.Stride3(1 << 30, 1 << 24, 64), s, s)
    assert f8(strides=bad8) == _lib.FA_ERR_UNSUPPORTED
    assert f8(strides=huge) == _lib.FA_ERR_UNSUPPORTED
    del ok


def test_fp8_binding_checks_without_gpu():
    q = torch.zeros(1, 16, 2, 64, dtype=torch.uint8)
    with pytest.raises(fa.FaArgError, match="float8"):
        fa.fwd_fp8(q.to(torch.bfloat16), q, q)
    with pytest.raises(fa.FaArgError, match="head_dim"):
        fa.fwd_fp8(*(torch.zeros(1, 16, 2, 32, dtype=torch.uint8),) * 3)
    with pytest.raises(fa.FaArgError, match="GPU"):
        fa.fwd_fp8(q, q.view(torch.float8_e4m3fn), q)
    with pytest.raises(fa.FaArgError, match="differ"):
        fa.fwd_fp8(q, torch.zeros(1, 16, 3, 64, dtype=torch.uint8),
                   torch.zeros(1, 16, 3, 64, dtype=torch.uint8))


def test_split_entry_points_without_launch():
    """fa_fwd_split's host functions and argument errors.  Every call of
    fa_fwd_split below is rejected before any HIP call (4096 keys with two
    splits leave two key ranges, so the workspace is required)."""
    lib = _lib.load()
    a256 = lambda x: (x + 255) // 256 * 256
    rows = 4 * 1 * 2 * 3  # S * B * H * Nq
    assert lib.fa_fwd_split_workspace_bytes(1, 2, 3, 64, 4) == a256(4 * rows * 64) + a256(4 * rows)
    for bad in [(1, 2, 3, 64, 0), (1, 2, 3, 64, 257), (1, 2, 3, 48, 2), (0, 2, 3, 64, 2)]:
        assert lib.fa_fwd_split_workspace_bytes(*bad) == 0

    # Split counts: launches with more than one wave per SIMD are not split
    # (the four sweep workloads; head_dim-128 key-group forms count twice);
    # narrow launches get splits of at least 2048 (or 1024) keys.
    assert lib.fa_fwd_split_count(1, 16, 16384, 16384, 64, 1) == 1
    assert lib.fa_fwd_split_count(1, 8, 8192, 8192, 128, 1) == 1
    assert lib.fa_fwd_split_count(2, 12, 2048, 2048, 64, 0) == 1
    assert lib.fa_fwd_split_count(2, 12, 512, 512, 64, 0) == 1
    assert lib.fa_fwd_split_count(1, 8, 4096, 4096, 128, 1) == 1
    assert lib.fa_fwd_split_count(1, 2, 16384, 16384, 64, 1) == 4
    # Splits of at least 2048 keys towards four waves per SIMD; where those
    # leave fewer than 1024 waves, splits down to 1024 keys up to 1024 waves.
    assert lib.fa_fwd_split_count(1, 16, 64, 16384, 64, 1) == 16
    assert lib.fa_fwd_split_count(1, 16, 65, 16384, 64, 1) == 16
    assert lib.fa_fwd_split_count(1, 16, 3, 16384, 64, 1) == 16
    assert lib.fa_fwd_split_count(1, 8, 128, 32768, 128, 1) == 32
    assert lib.fa_fwd_split_count(1, 12, 512, 4096, 64, 0) == 4
    assert lib.fa_fwd_split_count(1, 16, 512, 16384, 64, 1) == 8
    assert lib.fa_fwd_split_count(1, 32, 512, 8192, 128, 1) == 4
    assert lib.fa_fwd_split_count(1, 16, 2048, 16384, 64, 1) == 4
    assert lib.fa_fwd_split_count(2, 8, 2048, 2048, 64, 0) == 1
    assert lib.fa_fwd_split_count(1, 8, 2048, 2048, 64, 0) == 2
    # One or two rows (the vector-unit kernel): 256 workgroups of at least
    # 1024 keys, none once B*H reaches 256.
    assert lib.fa_fwd_split_count(1, 16, 1, 16384, 64, 1) == 16
    assert lib.fa_fwd_split_count(1, 8, 2, 32768, 128, 0) == 32
    assert lib.fa_fwd_split_count(1, 32, 2, 8192, 128, 1) == 8
    assert lib.fa_fwd_split_count(8, 8, 1, 8192, 128, 1) == 4
    assert lib.fa_fwd_split_count(1, 8, 1, 3000, 128, 1) == 2
    assert lib.fa_fwd_split_count(16, 16, 1, 65536, 64, 1) == 1
    assert lib.fa_fwd_split_count(1, 1, 2, 1 << 20, 64, 0) == 64
    assert lib.fa_fwd_split_count(1, 16, 1, 2048, 64, 1) == 2
    assert lib.fa_fwd_split_count(1, 16, 1, 1023, 64, 1) == 1
    assert lib.fa_fwd_split_count(1, 1, 1, 500, 64, 0) == 1
    assert lib.fa_fwd_split_count(0, 1, 1, 500, 64, 0) == 1

    need = lib.fa_fwd_split_workspace_bytes(1, 1, 128, 64, 2)

    def split(S=2, ws=P, wsb=1 << 40, Nq=128, Nk=4096, D=64):
        return lib.fa_fwd_split(P, P, P, P, P, 1, 1, Nq, Nk, D, 0, 0.125, _lib.FA_BF16, None,
                                S, ws, wsb, None)

    assert split(S=0) == _lib.FA_ERR_INVALID_ARG
    assert split(S=257) == _lib.FA_ERR_INVALID_ARG
    assert split(ws=None) == _lib.FA_ERR_INVALID_ARG
    assert split(wsb=need - 1) == _lib.FA_ERR_INVALID_ARG
    assert split(ws=P + 16) == _lib.FA_ERR_UNSUPPORTED
    assert split(D=48) == _lib.FA_ERR_UNSUPPORTED
    assert split(Nq=0) == _lib.FA_ERR_INVALID_ARG


def test_huge_sizes_do_not_overflow():
    """Size products near the int range are rejected (or give 0 / 1) without
    any intermediate overflow: B*H*N is compared by division first."""
    lib = _lib.load()
    big = (1 << 31) - 1
    assert lib.fa_fwd_split_count(1 << 30, big, 4114, 129, 128, 1) == 1
    assert lib.fa_fwd_split_workspace_bytes(big, big, big, 64, 2) == 0
    assert lib.fa_bwd_qk_workspace_bytes(big, big, 2, 2, 64) == 0
    assert lib.fa_bwd_qk_workspace_bytes(1, 1, 5, 5, 48) == 0
    assert lib.fa_fwd_qk(P, P, P, P, P, big, big, big, big, 64, 0, 0.125, _lib.FA_BF16, None,
                         None) == _lib.FA_ERR_UNSUPPORTED
    assert lib.fa_merge(P, P, big, P, P, 1 << 15, 1 << 15, 1, 64, _lib.FA_BF16,
                        None) == _lib.FA_ERR_UNSUPPORTED


def test_noalloc_rejects_before_launch():
    """fa_bwd_noalloc validates like fa_bwd_qk, and a problem whose backward
    scratch exceeds the static array's size is refused with FA_ERR_TOO_LARGE,
    all before any HIP call (none is made here: no device is needed)."""
    lib = _lib.load()
    cap = int(lib.fa_bwd_noalloc_max_bytes())
    assert cap == 64 << 20

    def call(ptrs=None, B=1, H=1, Nq=128, Nk=128, D=64, causal=0, scale=0.125,
             dtype=_lib.FA_BF16, strides=None):
        ptrs = [P] * 9 if ptrs is None else ptrs
        return lib.fa_bwd_noalloc(*ptrs, B, H, Nq, Nk, D, causal, scale, dtype, strides, None)

    for i in range(9):
        ptrs = [P] * 9
        ptrs[i] = None
        assert call(ptrs=ptrs) == _lib.FA_ERR_INVALID_ARG, i
    assert call(D=80) == _lib.FA_ERR_UNSUPPORTED
    assert call(causal=2) == _lib.FA_ERR_INVALID_ARG
    assert call(scale=float("nan")) == _lib.FA_ERR_INVALID_ARG
    assert call(B=0) == _lib.FA_ERR_INVALID_ARG
    # Largest N whose non-causal scratch fits, and the next size up.
    fits = [n for n in (8192, 16384)
            if lib.fa_bwd_qk_workspace_bytes_for(1, 8, n, n, 128, 0) <= cap]
    assert fits == [8192]
    assert call(B=1, H=16, Nq=16384, Nk=16384, D=64, causal=1) == _lib.FA_ERR_TOO_LARGE
    assert call(B=1, H=8, Nq=16384, Nk=16384, D=128) == _lib.FA_ERR_TOO_LARGE
    # The causal B1 H8 N8192 D128 backward splits its 32 key blocks per head
    # into 2 query segments, whose fp32 partial dK, dV sums (128 MiB) exceed
    # the array.
    assert lib.fa_bwd_qk_workspace_bytes_for(1, 8, 8192, 8192, 128, 1) > cap
    assert call(B=1, H=8, Nq=8192, Nk=8192, D=128, causal=1) == _lib.FA_ERR_TOO_LARGE
    assert b"TOO_LARGE" in lib.fa_status_str(_lib.FA_ERR_TOO_LARGE)


def _device_visible() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_device_visible(), reason="needs a host without a visible GPU: the "
                    "arguments are valid but the pointers are not device memory")
def test_hip_error_without_device():
    """With valid arguments and no device, every entry point that launches
    returns FA_ERR_HIP (the launch, or the device lookup of the no-alloc
    backward, fails), instead of crashing or reporting success."""
    lib = _lib.load()
    bf = _lib.FA_BF16
    assert lib.fa_fwd(P, P, P, P, P, 1, 1, 128, 64, 0, 0.125, bf, None, None) == _lib.FA_ERR_HIP
    assert lib.fa_fwd_qk(P, P, P, P, P, 1, 1, 64, 128, 128, 1, 0.1, bf, None,
                         None) == _lib.FA_ERR_HIP
    assert lib.fa_bwd(*([P] * 9), 1, 1, 128, 64, 0, 0.125, bf, None, P, 1 << 30,
                      None) == _lib.FA_ERR_HIP
    assert lib.fa_bwd_noalloc(*([P] * 9), 1, 1, 128, 128, 64, 0, 0.125, bf, None,
                              None) == _lib.FA_ERR_HIP
    assert lib.fa_merge(P, P, 2, P, P, 1, 1, 64, 64, bf, None) == _lib.FA_ERR_HIP
    assert lib.fa_fwd_fp8(P, P, P, P, P, None, None, None, 1, 1, 128, 128, 64, 0, 0.125, bf,
                          None, None) == _lib.FA_ERR_HIP
    assert lib.fa_fwd_split(P, P, P, P, P, 1, 1, 1, 8192, 64, 1, 0.125, bf, None, 4, P,
                            1 << 30, None) == _lib.FA_ERR_HIP
    assert b"HIP" in lib.fa_status_str(_lib.FA_ERR_HIP)

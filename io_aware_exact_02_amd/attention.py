"""Python binding of libfa: fused exact attention on MI355X.

Argument marshalling only.  torch supplies device memory and the current
stream; every step of the computation runs in libfa's HIP kernels.  There
is no fallback path: if libfa.so is missing the first call raises.

API names follow the pages' usage: ``flash_attn_func(q, k, v, causal)`` on
``[batch, seq, heads, head_dim]`` tensors (hotelren.com FlashAttention-2
walkthrough, sections 4 and 5) and ``flash_attn_qkvpacked_func(qkv)`` on a
packed ``[B, N, 3, H, D]`` tensor (bjdmk.com.cn page, section "实战集成").
Inputs must be fp16 or bf16 -- fp32 is rejected, as the walkthrough's
section 5 notes for the original library.
"""

from __future__ import annotations

import ctypes
import math

import torch

from . import _lib

_DTYPES = {torch.float16: _lib.FA_F16, torch.bfloat16: _lib.FA_BF16}


class FaArgError(ValueError):
    """An argument the library rejects (shape, dtype, device, layout)."""


def _check_inputs(*tensors):
    t0 = tensors[0]
    if t0.dim() != 4:
        raise FaArgError(f"expected [batch, seq, heads, head_dim] tensors, got {tuple(t0.shape)}")
    if t0.dtype not in _DTYPES:
        raise FaArgError(f"only float16 / bfloat16 inputs are supported, got {t0.dtype}")
    for t in tensors[1:]:
        if t.shape != t0.shape:
            raise FaArgError(f"shape mismatch: {tuple(t.shape)} vs {tuple(t0.shape)}")
        if t.dtype != t0.dtype:
            raise FaArgError(f"dtype mismatch: {t.dtype} vs {t0.dtype}")
        if t.device != t0.device:
            raise FaArgError(f"device mismatch: {t.device} vs {t0.device}")
    B, N, H, D = t0.shape
    if D not in (64, 128):
        raise FaArgError(f"head_dim must be 64 or 128, got {D}")
    if t0.device.type != "cuda":
        raise FaArgError(f"inputs must be on a GPU device, got {t0.device}")
    return B, N, H, D


def _check_qkv(q, k, v):
    """q [B, Nq, H, D] against k, v [B, Nk, H, D]; returns (B, Nq, Nk, H, D)."""
    for t in (q, k, v):
        if t.dim() != 4:
            raise FaArgError(f"expected [batch, seq, heads, head_dim] tensors, got {tuple(t.shape)}")
    if k.shape != v.shape:
        raise FaArgError(f"shape mismatch: {tuple(v.shape)} vs {tuple(k.shape)}")
    if (q.shape[0], q.shape[2], q.shape[3]) != (k.shape[0], k.shape[2], k.shape[3]):
        raise FaArgError(f"q {tuple(q.shape)} and k, v {tuple(k.shape)} differ in batch, heads "
                         "or head_dim")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise FaArgError(f"dtype mismatch: {q.dtype}, {k.dtype}, {v.dtype}")
    if q.device != k.device or q.device != v.device:
        raise FaArgError(f"device mismatch: {q.device}, {k.device}, {v.device}")
    B, Nq, H, D = _check_inputs(q)
    return B, Nq, k.shape[1], H, D


def _usable(t: torch.Tensor) -> torch.Tensor:
    """The kernels need d-stride 1, b/n/h strides that are multiples of 8
    elements and a 16-byte aligned base; copy otherwise."""
    s = t.stride()
    if s[3] != 1 or any(x % 8 for x in s[:3]) or t.data_ptr() % 16:
        return t.contiguous()
    return t


def _stride3(t: torch.Tensor) -> _lib.Stride3:
    s = t.stride()
    return _lib.Stride3(s[0], s[1], s[2])


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _scale(softmax_scale, D):
    return 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)


def _raise(status: int, what: str):
    msg = _lib.load().fa_status_str(status).decode()
    if status in (_lib.FA_ERR_INVALID_ARG, _lib.FA_ERR_UNSUPPORTED):
        raise FaArgError(f"{what}: {msg}")
    raise RuntimeError(f"{what}: {msg}")


def fwd(q, k, v, causal: bool = False, softmax_scale=None, out=None, lse=None,
        num_splits=None):
    """Forward pass.  q [B,Nq,H,D], k and v [B,Nk,H,D] (Nk = Nq for
    self-attention).  Returns (o [B,Nq,H,D], lse [B,H,Nq] fp32).  With
    Nq != Nk the causal mask is aligned to the last query and key.

    num_splits: key splits (fa_fwd_split); None picks fa_fwd_split_count's
    choice, 1 keeps the whole key range in each workgroup."""
    lib = _lib.load()
    B, N, Nk, H, D = _check_qkv(q, k, v)
    q, k, v = _usable(q), _usable(k), _usable(v)
    if out is None:
        out = torch.empty((B, N, H, D), dtype=q.dtype, device=q.device)
    else:
        _check_inputs(q, out)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    elif lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise FaArgError("lse must be a contiguous float32 [B, H, N] tensor")
    if num_splits is None:
        num_splits = lib.fa_fwd_split_count(B, H, N, Nk, D, int(bool(causal)))
    elif not isinstance(num_splits, int) or not 1 <= num_splits <= 256:
        raise FaArgError(f"num_splits must be an int in 1..256, got {num_splits!r}")
    out_u = _usable(out)
    st = _lib.FwdStrides(_stride3(q), _stride3(k), _stride3(v), _stride3(out_u))
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out_u.data_ptr(), lse.data_ptr(), B, H, N,
            Nk, D, int(bool(causal)), _scale(softmax_scale, D), _DTYPES[q.dtype],
            ctypes.byref(st))
    if num_splits > 1:
        nbytes = int(lib.fa_fwd_split_workspace_bytes(B, H, N, D, num_splits))
        ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
        status = lib.fa_fwd_split(*args, num_splits, ws.data_ptr(), nbytes, _stream(q))
        what = "fa_fwd_split"
    else:
        status = lib.fa_fwd_qk(*args, _stream(q))
        what = "fa_fwd_qk"
    if status != _lib.FA_OK:
        _raise(status, what)
    if out_u is not out:
        out.copy_(out_u)
    return out, lse


_FP8_DTYPES = (torch.float8_e4m3fn, torch.uint8)


def _usable8(t: torch.Tensor) -> torch.Tensor:
    """8-bit rows must start 16-byte aligned: d-stride 1, b/n/h strides that
    are multiples of 16 bytes (n stride below 2^24) and a 16-byte aligned
    base; copy otherwise."""
    s = t.stride()
    if s[3] != 1 or any(x % 16 for x in s[:3]) or s[1] >= 1 << 24 or t.data_ptr() % 16:
        return t.contiguous()
    return t


def _descale(x, B: int, H: int, device) -> torch.Tensor | None:
    if x is None:
        return None
    if not isinstance(x, torch.Tensor):
        return torch.full((B, H), float(x), dtype=torch.float32, device=device)
    if x.dtype != torch.float32 or x.device != device or x.numel() != B * H:
        raise FaArgError(f"descale factors must be float32 [B, H] = [{B}, {H}] on {device}, "
                         f"got {x.dtype} {tuple(x.shape)} on {x.device}")
    return x.reshape(B, H).contiguous()


def fwd_fp8(q, k, v, descale_q=None, descale_k=None, descale_v=None, causal: bool = False,
            softmax_scale=None, out_dtype=torch.bfloat16, out=None, lse=None):
    """Forward pass with FP8 inputs.  q [B,Nq,H,D], k and v [B,Nk,H,D] hold
    OCP E4M3 codes (torch.float8_e4m3fn, or uint8 with the same bits); the
    optional descale factors (float32 [B, H] tensors or Python floats, None
    for 1) give the values descale * e4m3(code).  Returns (o [B,Nq,H,D] in
    ``out_dtype`` (bfloat16 or float16), lse [B,H,Nq] fp32)."""
    lib = _lib.load()
    for t in (q, k, v):
        if t.dim() != 4:
            raise FaArgError(f"expected [batch, seq, heads, head_dim] tensors, got {tuple(t.shape)}")
        if t.dtype not in _FP8_DTYPES:
            raise FaArgError(f"fwd_fp8 takes float8_e4m3fn (or uint8) codes, got {t.dtype}")
        if t.device != q.device:
            raise FaArgError(f"device mismatch: {t.device} vs {q.device}")
    if k.shape != v.shape:
        raise FaArgError(f"shape mismatch: {tuple(v.shape)} vs {tuple(k.shape)}")
    if (q.shape[0], q.shape[2], q.shape[3]) != (k.shape[0], k.shape[2], k.shape[3]):
        raise FaArgError(f"q {tuple(q.shape)} and k, v {tuple(k.shape)} differ in batch, heads "
                         "or head_dim")
    B, N, H, D = q.shape
    Nk = k.shape[1]
    if D not in (64, 128):
        raise FaArgError(f"head_dim must be 64 or 128, got {D}")
    if q.device.type != "cuda":
        raise FaArgError(f"inputs must be on a GPU device, got {q.device}")
    if out_dtype not in _DTYPES:
        raise FaArgError(f"out_dtype must be float16 or bfloat16, got {out_dtype}")
    q, k, v = (_usable8(t.view(torch.uint8)) for t in (q, k, v))
    ds = [_descale(x, B, H, q.device) for x in (descale_q, descale_k, descale_v)]
    if out is None:
        out = torch.empty((B, N, H, D), dtype=out_dtype, device=q.device)
    elif out.shape != (B, N, H, D) or out.dtype != out_dtype or out.device != q.device:
        raise FaArgError("out must be a [B, Nq, H, D] tensor of out_dtype on the inputs' device")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    elif lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise FaArgError("lse must be a contiguous float32 [B, H, N] tensor")
    out_u = _usable(out)
    st = _lib.FwdStrides(_stride3(q), _stride3(k), _stride3(v), _stride3(out_u))
    ptr = lambda t: None if t is None else t.data_ptr()
    status = lib.fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out_u.data_ptr(),
                            lse.data_ptr(), ptr(ds[0]), ptr(ds[1]), ptr(ds[2]), B, H, N, Nk, D,
                            int(bool(causal)), _scale(softmax_scale, D), _DTYPES[out_dtype],
                            ctypes.byref(st), _stream(q))
    if status != _lib.FA_OK:
        _raise(status, "fa_fwd_fp8")
    if out_u is not out:
        out.copy_(out_u)
    return out, lse


def workspace_bytes(B: int, H: int, N: int, D: int, Nk: int | None = None,
                    causal: bool | None = None) -> int:
    """Backward workspace for N query rows against Nk (default N) keys: the
    size one mask needs, or (causal=None) the size that serves either."""
    lib = _lib.load()
    nk = N if Nk is None else Nk
    if causal is None:
        return int(lib.fa_bwd_qk_workspace_bytes(B, H, N, nk, D))
    return int(lib.fa_bwd_qk_workspace_bytes_for(B, H, N, nk, D, int(bool(causal))))


def bwd(q, k, v, o, lse, dout, causal: bool = False, softmax_scale=None,
        dq=None, dk=None, dv=None, workspace=None, stage_hook=None):
    """Backward pass.  Returns (dq [B,Nq,H,D], dk, dv [B,Nk,H,D]) in the
    input type.

    ``stage_hook``: optional callable; when given, the three backward kernels
    are enqueued one by one and ``stage_hook(name)`` is called before and
    after the dK/dV stage with name "dkdv_begin" / "dkdv_end" (used to record
    stream events around that kernel).
    """
    lib = _lib.load()
    B, N, Nk, H, D = _check_qkv(q, k, v)
    _check_inputs(q, o, dout)
    q, k, v, o, dout = (_usable(t) for t in (q, k, v, o, dout))
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise FaArgError("lse must be a contiguous float32 [B, H, N] tensor")
    if dq is None:
        dq = torch.empty((B, N, H, D), dtype=q.dtype, device=q.device)
    if dk is None:
        dk = torch.empty((B, Nk, H, D), dtype=q.dtype, device=q.device)
    if dv is None:
        dv = torch.empty((B, Nk, H, D), dtype=q.dtype, device=q.device)
    _check_inputs(q, dq)
    _check_inputs(k, dk, dv)
    need = lib.fa_bwd_qk_workspace_bytes_for(B, H, N, Nk, D, int(bool(causal)))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = _lib.BwdStrides(*(_stride3(t) for t in (q, k, v, o, dout, dq, dk, dv)))
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, Nk, D,
            int(bool(causal)), _scale(softmax_scale, D), _DTYPES[q.dtype], ctypes.byref(st),
            workspace.data_ptr(), workspace.numel() * workspace.element_size())
    if stage_hook is None:
        status = lib.fa_bwd_qk(*args, _lib.STAGE_ALL, _stream(q))
        if status != _lib.FA_OK:
            _raise(status, "fa_bwd_qk")
        return dq, dk, dv
    for stage in (_lib.STAGE_PREPROCESS, _lib.STAGE_DKDV, _lib.STAGE_DQ):
        if stage == _lib.STAGE_DKDV:
            stage_hook("dkdv_begin")
        status = lib.fa_bwd_qk(*args, stage, _stream(q))
        if status != _lib.FA_OK:
            _raise(status, "fa_bwd_qk")
        if stage == _lib.STAGE_DKDV:
            stage_hook("dkdv_end")
    return dq, dk, dv


def merge(o_parts, lse_parts):
    """Exact merge of results over disjoint key sets (fa_merge).

    o_parts [P, B, N, H, D] (dtype) and lse_parts [P, B, H, N] (fp32), for
    example torch.stack of several fwd results.  Returns (o [B,N,H,D],
    lse [B,H,N])."""
    lib = _lib.load()
    if o_parts.dim() != 5 or lse_parts.dim() != 4:
        raise FaArgError("expected o_parts [P, B, N, H, D] and lse_parts [P, B, H, N]")
    P, B, N, H, D = o_parts.shape
    if tuple(lse_parts.shape) != (P, B, H, N) or lse_parts.dtype != torch.float32:
        raise FaArgError(f"lse_parts must be float32 [P, B, H, N] = {(P, B, H, N)}")
    _check_inputs(o_parts[0])
    if lse_parts.device != o_parts.device:
        raise FaArgError("o_parts and lse_parts must be on one device")
    o_parts, lse_parts = o_parts.contiguous(), lse_parts.contiguous()
    o = torch.empty((B, N, H, D), dtype=o_parts.dtype, device=o_parts.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=o_parts.device)
    status = lib.fa_merge(o_parts.data_ptr(), lse_parts.data_ptr(), P, o.data_ptr(),
                          lse.data_ptr(), B, H, N, D, _DTYPES[o_parts.dtype], _stream(o))
    if status != _lib.FA_OK:
        _raise(status, "fa_merge")
    return o, lse


class _FlashAttn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal, softmax_scale):
        o, lse = fwd(q, k, v, causal, softmax_scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal = causal
        ctx.softmax_scale = softmax_scale
        return o

    @staticmethod
    def backward(ctx, dout):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = bwd(q, k, v, o, lse, _usable(dout), ctx.causal, ctx.softmax_scale)
        return dq, dk, dv, None, None


class _FlashAttnQKVPacked(torch.autograd.Function):
    @staticmethod
    def forward(ctx, qkv, causal, softmax_scale):
        q, k, v = qkv.unbind(dim=2)
        o, lse = fwd(q, k, v, causal, softmax_scale)
        ctx.save_for_backward(qkv, o, lse)
        ctx.causal = causal
        ctx.softmax_scale = softmax_scale
        return o

    @staticmethod
    def backward(ctx, dout):
        qkv, o, lse = ctx.saved_tensors
        q, k, v = qkv.unbind(dim=2)
        dqkv = torch.empty_like(qkv)
        dq, dk, dv = dqkv.unbind(dim=2)
        bwd(q, k, v, o, lse, _usable(dout), ctx.causal, ctx.softmax_scale, dq=dq, dk=dk, dv=dv)
        return dqkv, None, None


def flash_attn_func(q, k, v, causal: bool = False, softmax_scale=None):
    """Exact attention on [B, N, H, D] tensors, differentiable.  k and v may
    have a different sequence length from q (causal mask aligned to the last
    query and key)."""
    return _FlashAttn.apply(q, k, v, causal, softmax_scale)


def flash_attn_qkvpacked_func(qkv, causal: bool = False, softmax_scale=None):
    """Exact attention on a packed [B, N, 3, H, D] tensor; returns [B, N, H, D].
    The gradient lands in one packed dqkv tensor (no copies of q, k, v)."""
    if qkv.dim() != 5 or qkv.shape[2] != 3:
        raise FaArgError(f"expected qkv of shape [B, N, 3, H, D], got {tuple(qkv.shape)}")
    return _FlashAttnQKVPacked.apply(qkv, causal, softmax_scale)

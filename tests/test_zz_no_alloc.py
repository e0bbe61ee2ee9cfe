"""fa_bwd_noalloc (the backward with its scratch in a static device array,
for callers that cannot allocate) against fa_bwd_qk with a caller workspace:
the same kernels on the same inputs, so dq, dk and dv must be equal bit for
bit.  Two calls in a row, the second smaller, so the second runs over the
scratch contents the first left behind."""

import ctypes

import pytest
import torch

from io_aware_exact_02_amd import _lib
from workloads import random_qkv

CASES = [
    # (B, H, Nq, Nk, D, causal, dtype): first a larger problem, then a smaller one
    (2, 4, 1000, 1000, 64, 1, "bf16"),
    (1, 3, 333, 500, 128, 0, "f16"),
]


def _inputs(B, H, Nq, Nk, D, dtype, seed):
    dev = torch.device("cuda")
    qa = random_qkv(B, Nq, H, D, dtype, seed)
    ka = random_qkv(B, Nk, H, D, dtype, seed + 1)
    q, k, v = qa["q"].to(dev), ka["k"].to(dev), ka["v"].to(dev)
    dout = qa["do"].to(dev)
    return q, k, v, dout


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


@pytest.mark.gpu
def test_noalloc_matches_workspace_backward_twice():
    import io_aware_exact_02_amd as fa
    lib = _lib.load()
    dev = torch.device("cuda")
    for i, (B, H, Nq, Nk, D, causal, dtype) in enumerate(CASES):
        print(f"noalloc case {i}: B={B} H={H} Nq={Nq} Nk={Nk} D={D} causal={causal} {dtype}",
              flush=True)
        q, k, v, dout = _inputs(B, H, Nq, Nk, D, dtype, 8800 + 10 * i)
        o, lse = fa.fwd(q, k, v, causal=bool(causal))
        scale = 1.0 / D ** 0.5
        dt = _lib.FA_BF16 if dtype == "bf16" else _lib.FA_F16
        ref = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
        got = [torch.full_like(q, float("nan")), torch.full_like(k, float("nan")),
               torch.full_like(v, float("nan"))]
        ws = torch.empty(int(lib.fa_bwd_qk_workspace_bytes(B, H, Nq, Nk, D)), dtype=torch.uint8,
                         device=dev)
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.fa_bwd_qk(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                           *(_ptr(t) for t in ref), B, H, Nq, Nk, D, causal, scale, dt, None,
                           _ptr(ws), ws.numel(), _lib.STAGE_ALL, ctypes.c_void_p(stream))
        assert st == _lib.FA_OK
        st = lib.fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                *(_ptr(t) for t in got), B, H, Nq, Nk, D, causal, scale, dt,
                                None, ctypes.c_void_p(stream))
        assert st == _lib.FA_OK
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), (i, name, float((a.float() - b.float()).abs().max()))
        assert all(torch.isfinite(t).all() for t in got)

"""Seeded synthetic inputs for the attention hot path.

This module only draws random numbers and arranges them in the layouts the
attention API takes.  It holds none of the attention arithmetic, so both the
HIP path (through the Python binding) and the CPU oracle can be fed from it
without sharing any code of the method.

Inputs follow the pages' own workloads: every example on them draws
Q, K, V with ``torch.randn`` in half precision (the qkv-packed example on the
bjdmk.com.cn page, section "实战集成"; the unfused-vs-fused comparison on the
pwwt.cn page, section "实战代码对比"; the benchmark on the hotelren.com
FlashAttention-2 walkthrough, section 4).  Values are drawn in float32 from a
seeded CPU generator and cast to the half type with round-to-nearest-even, so
the GPU and the oracle receive exactly the same bit patterns.
"""

from __future__ import annotations

import dataclasses

import math

import torch

DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention problem: sizes, element type, mask and memory layout.

    ``layout`` is ``"bnhd"`` (separate q, k, v in ``[B, N, H, D]``) or
    ``"packed"`` (one ``qkv`` tensor ``[B, N, 3, H, D]`` whose slices are
    strided views).
    """

    name: str
    B: int
    H: int
    N: int
    D: int
    dtype: str
    causal: bool
    layout: str
    seed: int

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    def describe(self) -> str:
        lay = "packed qkv [B,N,3,H,D]" if self.layout == "packed" else "[B,N,H,D]"
        return (f"B={self.B} H={self.H} N={self.N} D={self.D} {self.dtype} "
                f"{lay} {'causal' if self.causal else 'non-causal'}")


# The five workloads the hot path is checked and measured on.
WORKLOADS = {
    "c1": Workload("c1", 1, 1, 128, 64, "bf16", False, "bnhd", 1001),
    "c2": Workload("c2", 2, 12, 512, 64, "f16", False, "packed", 1002),
    "c3": Workload("c3", 2, 12, 2048, 64, "f16", False, "packed", 1003),
    "c4": Workload("c4", 1, 8, 8192, 128, "bf16", True, "bnhd", 1004),
    "c5": Workload("c5", 1, 16, 16384, 64, "bf16", True, "bnhd", 1005),
}


# The speed sweep of the hotelren.com FlashAttention-2 walkthrough, section
# 4: B=2, H=8, D=64, fp16 q, k, v in [B, N, H, D] at N = 2048, 4096 and 8192
# (non-causal), plus the causal run at N = 4096.
PAGES_SWEEP = {
    "s2048": Workload("s2048", 2, 8, 2048, 64, "f16", False, "bnhd", 1102),
    "s4096": Workload("s4096", 2, 8, 4096, 64, "f16", False, "bnhd", 1104),
    "s8192": Workload("s8192", 2, 8, 8192, 64, "f16", False, "bnhd", 1108),
    "s4096c": Workload("s4096c", 2, 8, 4096, 64, "f16", True, "bnhd", 1114),
}


# Shapes for profiling the workgroup -> XCD mapping: 12 heads, a count the
# eight XCDs do not divide (each XCD's L2 serves two of them rather than
# three), causal, at head_dim 64 and 128.
PROFILE_SHAPES = {
    "h12": Workload("h12", 1, 12, 8192, 64, "bf16", True, "bnhd", 1212),
    "h12d128": Workload("h12d128", 1, 12, 8192, 128, "bf16", True, "bnhd", 1213),
}


def _randn(shape, gen: torch.Generator, dtype: torch.dtype) -> torch.Tensor:
    return torch.randn(shape, dtype=torch.float32, generator=gen).to(dtype)


def make_inputs(w: Workload, dout: str = "randn") -> dict:
    """Draw q, k, v and dO for ``w`` on the CPU.

    Draw order is q, k, v (or the single packed qkv), then dO.  ``dout`` is
    ``"randn"`` (N(0,1)) or ``"ones"`` (the ``out.sum()`` loss of the
    qkv-packed example).  Returns CPU tensors; ``q``, ``k``, ``v`` are views
    into ``qkv`` when the layout is packed.
    """
    gen = torch.Generator("cpu").manual_seed(w.seed)
    dt = w.torch_dtype
    out = {}
    if w.layout == "packed":
        qkv = _randn((w.B, w.N, 3, w.H, w.D), gen, dt)
        out["qkv"] = qkv
        out["q"], out["k"], out["v"] = qkv.unbind(dim=2)
    elif w.layout == "bnhd":
        for name in ("q", "k", "v"):
            out[name] = _randn((w.B, w.N, w.H, w.D), gen, dt)
    else:
        raise ValueError(f"unknown layout {w.layout!r}")
    if dout == "randn":
        out["do"] = _randn((w.B, w.N, w.H, w.D), gen, dt)
    elif dout == "ones":
        out["do"] = torch.ones((w.B, w.N, w.H, w.D), dtype=dt)
    else:
        raise ValueError(f"unknown dout {dout!r}")
    return out


def random_qkv(B: int, N: int, H: int, D: int, dtype: str, seed: int,
               layout: str = "bnhd") -> dict:
    """Same recipe for an arbitrary (small or odd) shape."""
    w = Workload("adhoc", B, H, N, D, dtype, False, layout, seed)
    return make_inputs(w)


def sample_rows(N: int, count: int, seed: int) -> list:
    """Query rows checked at full size when the oracle cannot cover all rows.

    Always includes the first and last rows and rows on both sides of the
    64-, 128- and N/2-boundaries; the rest are seeded uniform draws.
    """
    fixed = {0, 1, 63, 64, 127, 128, 129, N // 2 - 1, N // 2, N - 2, N - 1}
    fixed = {r for r in fixed if 0 <= r < N}
    gen = torch.Generator("cpu").manual_seed(seed)
    extra = torch.randperm(N, generator=gen).tolist()
    rows = sorted(fixed)
    for r in extra:
        if len(rows) >= count:
            break
        if r not in fixed:
            rows.append(r)
    return sorted(rows[:max(count, len(fixed))])


# ------------------------------------------------------------- FP8 inputs
#
# FP8 attention takes E4M3 codes plus one descale factor per (batch, head)
# for each of q, k, v (the value of code c is descale * e4m3(c)).  The
# inputs below are quantized here with torch's own float -> float8_e4m3fn
# conversion (round to nearest even); the codes travel as uint8 tensors.


def quantize_e4m3_per_head(x: torch.Tensor):
    """x [B, N, H, D] -> (codes uint8 [B, N, H, D], descale float32 [B, H]),
    descale = max|x| / 448 over each (batch, head)."""
    xf = x.float()
    amax = xf.abs().amax(dim=(1, 3)).clamp_min(1e-30)
    ds = amax / 448.0
    y = (xf / ds[:, None, :, None]).clamp(-448.0, 448.0)
    return y.to(torch.float8_e4m3fn).view(torch.uint8), ds


def fp8_random_inputs(B: int, Nq: int, Nk: int, H: int, D: int, seed: int,
                      per_head_scale: bool = True) -> dict:
    """N(0,1) q [B, Nq, H, D], k, v [B, Nk, H, D], each quantized per head
    (or, with per_head_scale=False, cast directly: descale factors of 1)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    out = {}
    for name, n in (("q", Nq), ("k", Nk), ("v", Nk)):
        x = torch.randn((B, n, H, D), dtype=torch.float32, generator=gen)
        if per_head_scale:
            out[name], out["descale_" + name] = quantize_e4m3_per_head(x)
        else:
            out[name] = x.to(torch.float8_e4m3fn).view(torch.uint8)
            out["descale_" + name] = torch.ones((B, H))
    return out


def fp8_exact_weight_inputs(B: int, Nq: int, Nk: int, H: int, D: int, seed: int) -> dict:
    """Inputs whose softmax weights are all powers of two.

    Each q row is +-1 at one random position (zero elsewhere), every k entry
    an integer in [-4, 4], so every raw score q.k is an integer in [-4, 4].
    With descale_q = 1/2, descale_k = 1/4 and scale = ln(2) / (1/2 * 1/4)
    the weight exp(scale * s) = 2^(raw score), and any weight taken relative
    to a reference point that is itself a raw score lies in [2^-8, 2^8], all
    exact in E4M3.  v is N(0,1) quantized per head.
    """
    gen = torch.Generator("cpu").manual_seed(seed)
    pos = torch.randint(0, D, (B, Nq, H), generator=gen)
    sign = torch.randint(0, 2, (B, Nq, H), generator=gen).float() * 2 - 1
    qv = torch.zeros((B, Nq, H, D))
    qv.scatter_(3, pos[..., None], sign[..., None])
    kv = torch.randint(-4, 5, (B, Nk, H, D), generator=gen).float()
    v = torch.randn((B, Nk, H, D), dtype=torch.float32, generator=gen)
    out = {"q": qv.to(torch.float8_e4m3fn).view(torch.uint8),
           "k": kv.to(torch.float8_e4m3fn).view(torch.uint8),
           "descale_q": torch.full((B, H), 0.5), "descale_k": torch.full((B, H), 0.25)}
    out["v"], out["descale_v"] = quantize_e4m3_per_head(v)
    out["scale"] = math.log(2.0) / (0.5 * 0.25)
    return out

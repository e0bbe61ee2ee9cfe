"""Multi-head attention layer around the fused kernel.

The FlashAttention IO-awareness article at 0539edu.com (section
"快速集成指南", the quick-integration guide) names a FlashMHA module that
takes the place of a standard multi-head attention layer as a whole.  This is that layer on top of libfa: one packed
QKV projection, exact attention through ``flash_attn_qkvpacked_func`` (the
HIP kernels, no copies of q, k, v), and an output projection.  The two
projections are plain library GEMMs (torch ``nn.Linear``); the attention
step runs only in libfa.  Weights are randomly initialised (no trained
weights are used anywhere here).
"""

from __future__ import annotations

import torch
from torch import nn

from .attention import FaArgError, flash_attn_qkvpacked_func


class FlashMHA(nn.Module):
    """Self-attention over x [B, N, embed_dim] -> [B, N, embed_dim].

    ``num_heads`` must give a head_dim of 64 or 128; ``causal`` applies the
    lower-triangular mask; ``softmax_scale`` defaults to 1/sqrt(head_dim).
    Parameters: ``Wqkv`` (embed_dim -> 3 * embed_dim, output ordered
    [q | k | v], each [heads, head_dim]) and ``out_proj``.
    """

    def __init__(self, embed_dim: int, num_heads: int, bias: bool = True, causal: bool = False,
                 softmax_scale=None, device=None, dtype=None):
        super().__init__()
        if embed_dim % num_heads:
            raise FaArgError(f"embed_dim {embed_dim} is not a multiple of num_heads {num_heads}")
        head_dim = embed_dim // num_heads
        if head_dim not in (64, 128):
            raise FaArgError(f"head_dim must be 64 or 128, got {head_dim}")
        self.embed_dim, self.num_heads, self.head_dim = embed_dim, num_heads, head_dim
        self.causal, self.softmax_scale = causal, softmax_scale
        kw = {"device": device, "dtype": dtype}
        self.Wqkv = nn.Linear(embed_dim, 3 * embed_dim, bias=bias, **kw)
        self.out_proj = nn.Linear(embed_dim, embed_dim, bias=bias, **kw)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        B, N, E = x.shape
        if E != self.embed_dim:
            raise FaArgError(f"expected embed_dim {self.embed_dim}, got {E}")
        qkv = self.Wqkv(x).view(B, N, 3, self.num_heads, self.head_dim)
        o = flash_attn_qkvpacked_func(qkv, causal=self.causal, softmax_scale=self.softmax_scale)
        return self.out_proj(o.reshape(B, N, E))

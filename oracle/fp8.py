"""FP8 (E4M3) attention forward for the oracle.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this module; only the tests use it.  It shares no code with the HIP
path.

The FlashAttention IO-awareness article at 0539edu.com (sections
"H100的FP8加速能力" and "未来展望：FlashAttention-3带来的新可能") says that
FlashAttention-3 takes FP8 inputs to raise throughput.  It gives no format,
scaling or rounding rule, so this module fixes the plainest reading:

* Inputs are OCP FP8 E4M3 codes: 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2^-6; the codes
  S.1111.111 are NaN and there are no infinities (largest finite value 448).
  Each of q, k, v comes with one float descale factor per (batch, head): the
  value of a code c is descale * e4m3(c).
* The result is exact attention over those values:
  O = softmax(scale * Q K^T) V and LSE as in ``oracle.attention``, with
  Q = descale_q * e4m3(q) and so on.
* The FP8 kernel rounds the softmax weights P to E4M3 before the second
  product (the only step on the path that is not exact up to fp32
  rounding) and normalises by the sum of the rounded weights.
  ``fp8_output_bound`` bounds the difference this makes, element by element.
"""

from __future__ import annotations

import numpy as np

from .attention import _head_rows, attention_forward, default_scale

E4M3_MAX = 448.0


def _codes(x) -> np.ndarray:
    """E4M3 codes as a uint8 numpy array (from numpy, or a torch uint8 or
    float8_e4m3fn tensor)."""
    if hasattr(x, "detach"):
        import torch
        t = x.detach().cpu()
        if t.dtype != torch.uint8:
            t = t.view(torch.uint8)
        return t.numpy()
    return np.asarray(x).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8 array or torch tensor), float64."""
    c = _codes(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def _descaled(codes, descale) -> np.ndarray:
    """codes [B, N, H, D], descale [B, H] -> float64 values."""
    ds = np.asarray(descale.detach().cpu().numpy() if hasattr(descale, "detach") else descale,
                    dtype=np.float64)
    return e4m3_decode(codes) * ds[:, None, :, None]


def attention_forward_fp8(q, k, v, descale_q, descale_k, descale_v, causal: bool = False,
                          scale: float | None = None):
    """O [B, Nq, H, D] and LSE [B, H, Nq] of exact attention over the
    descaled E4M3 inputs (codes [B, N, H, D], descales [B, H])."""
    return attention_forward(_descaled(q, descale_q), _descaled(k, descale_k),
                             _descaled(v, descale_v), causal=causal, scale=scale)


def _bound_rows(Q, K, V, rows, causal, scale, offset):
    """O, LSE and the output bound for query rows ``rows`` of one (batch,
    head): Q [R, D] the rows' query vectors, K, V [Nk, D] descaled values."""
    res = _head_rows(Q, K, V, rows, causal, scale, offset=offset)
    P, O = res["P"], res["O"]                                       # [R, Nk], [R, D]
    pmax = P.max(axis=1, keepdims=True) if P.shape[1] else np.zeros((P.shape[0], 1))
    visible = P > 0.0
    p = np.divide(P, pmax, out=np.zeros_like(P), where=pmax > 0)   # row max = 1
    e = np.where(visible, np.maximum(2.0 ** -4 * p, 2.0 ** -10) + 2.0 ** -12 * p, 0.0)
    low = np.maximum(p.sum(1) - e.sum(1), 1.0 - 2.0 ** -4 - 2.0 ** -12)  # [R]
    num = np.empty_like(O)
    for d in range(V.shape[1]):   # sum_j e_j |v_jd - O_id|, one d at a time
        num[:, d] = (e * np.abs(V[None, :, d] - O[:, d:d + 1])).sum(1)
    vmax = np.abs(V).max() if V.size else 0.0
    bound = num / low[:, None] + 2.0 ** -8 * np.abs(O) + 1e-4 * vmax
    bound = np.where(visible.any(1)[:, None], bound, 0.0)
    return O, res["LSE"], bound


def fp8_output_bound(q, k, v, descale_q, descale_k, descale_v, causal: bool = False,
                     scale: float | None = None):
    """Elementwise bound [B, Nq, H, D] on |O_kernel - O| for the FP8 kernel.

    Let p_j = exp(s_j - max s) be the exact weights of one row (largest 1)
    and p^_j the weights the kernel multiplies V by, taken in the same units.
    The kernel computes its weights against a reference point at or below the
    row maximum, so in its own units the largest weight is at least 1, and
    rounds each one to E4M3 (round to nearest): the error is at most half a
    unit in the last place, 2^-4 p relative for normal values and 2^-10
    absolute in the subnormal range.  Back in the row's units this gives
    |p^_j - p_j| <= e_j = max(2^-4 p_j, 2^-10) + 2^-12 p_j, where the last
    term covers the fp32 score and exp2 rounding ahead of the E4M3 rounding.
    With O = sum_j p_j v_j / sum_j p_j and the kernel's
    O^ = sum_j p^_j v_j / sum_j p^_j, exactly
        O^ - O = sum_j (p^_j - p_j) (v_j - O) / sum_j p^_j,
    and sum_j p^_j >= max(sum_j p_j - sum_j e_j, 1 - 2^-4 - 2^-12).  Added:
    2^-8 |O| for rounding the output to bf16 or fp16 and 1e-4 max|v| for the
    fp32 accumulation.  Keys the mask hides carry no weight on either side,
    and rows that see no key have a bound of 0 (both sides are exactly 0).
    """
    Q = _descaled(q, descale_q)
    K = _descaled(k, descale_k)
    V = _descaled(v, descale_v)
    B, N, H, D = Q.shape
    scale = default_scale(D) if scale is None else float(scale)
    rows = np.arange(N)
    out = np.zeros((B, N, H, D))
    for b in range(B):
        for h in range(H):
            out[b, :, h, :] = _bound_rows(Q[b, :, h, :], K[b, :, h, :], V[b, :, h, :], rows,
                                          causal, scale, K.shape[1] - N)[2]
    return out


def fp8_rows(q, k, v, descale_q, descale_k, descale_v, b: int, h: int, rows,
             causal: bool = False, scale: float | None = None):
    """O [R, D], LSE [R] and the output bound [R, D] at selected query rows of
    one (b, h), without forming the other rows."""
    rows = np.asarray(rows)
    ds = lambda x: np.asarray(x.detach().cpu().numpy() if hasattr(x, "detach") else x,
                              dtype=np.float64)[b, h]
    qc, kc, vc = _codes(q), _codes(k), _codes(v)
    Q = e4m3_decode(qc[b, rows, h, :]) * ds(descale_q)
    K = e4m3_decode(kc[b, :, h, :]) * ds(descale_k)
    V = e4m3_decode(vc[b, :, h, :]) * ds(descale_v)
    scale = default_scale(K.shape[1]) if scale is None else float(scale)
    O, LSE, bound = _bound_rows(Q, K, V, rows, causal, scale, kc.shape[1] - qc.shape[1])
    return {"O": O, "LSE": LSE, "bound": bound}

"""FP8 (E4M3) attention forward for the oracle.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this module; only the tests and the graft smoke check use it.  It
shares no code with the HIP path.

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

from .attention import attention_forward, attention_probs, default_scale

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8 array or torch uint8 tensor), float64."""
    if hasattr(codes, "detach"):
        codes = codes.detach().cpu().numpy()
    c = np.asarray(codes).astype(np.uint8).astype(np.int64)
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
    if scale is None:
        scale = default_scale(Q.shape[-1])
    O, _ = attention_forward(Q, K, V, causal=causal, scale=scale)
    P = attention_probs(Q, K, causal=causal, scale=scale)          # [B, H, Nq, Nk]
    pmax = P.max(axis=-1, keepdims=True)
    visible = P > 0.0
    p = np.divide(P, pmax, out=np.zeros_like(P), where=pmax > 0)   # row max = 1
    e = np.where(visible, np.maximum(2.0 ** -4 * p, 2.0 ** -10) + 2.0 ** -12 * p, 0.0)
    low = np.maximum(p.sum(-1) - e.sum(-1), 1.0 - 2.0 ** -4 - 2.0 ** -12)  # [B, H, Nq]
    Vh = np.transpose(V, (0, 2, 1, 3))                              # [B, H, Nk, D]
    Oh = np.transpose(O, (0, 2, 1, 3))                              # [B, H, Nq, D]
    # sum_j e_j |v_j - O_i| without forming [.., Nq, Nk, D]: split |a - b|
    # by the sign of v_j - O_i per d is not linear, so loop over d.
    num = np.empty_like(Oh)
    for d in range(Vh.shape[-1]):
        diff = np.abs(Vh[:, :, None, :, d] - Oh[:, :, :, None, d])  # [B, H, Nq, Nk]
        num[..., d] = (e * diff).sum(-1)
    vmax = np.abs(V).max(axis=(1, 3))                               # [B, H]
    bound = num / low[..., None] + 2.0 ** -8 * np.abs(Oh) + 1e-4 * vmax[:, :, None, None]
    empty = ~visible.any(-1)                                        # [B, H, Nq]
    bound = np.where(empty[..., None], 0.0, bound)
    return np.transpose(bound, (0, 2, 1, 3))

"""Plain float64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this module; only the tests, the smoke check
(``__graft_entry__.smoke``) and the ``cpu_baseline`` leg of ``bench.py`` use
it.  It shares no code with the HIP
path.

What it computes, and where the pages define it:

* Forward: ``O = softmax(scale * Q K^T) V`` with ``scale = 1/sqrt(D)`` by
  default -- the attention formula on the bjdmk.com.cn page (section
  "性能引擎：FlashAttention 如何重塑注意力计算？") and the three-step unfused
  code on the pwwt.cn page (section "FlashAttention 是如何做到又快又省内存的？").
  The fused method reaches exactly this result ("exact, not an
  approximation": bjdmk.com.cn, same section; hotelren.com FlashAttention-2
  walkthrough, section 5).
* The causal variant masks the upper triangle (keys j > query i): the
  "causal (lower-triangular) mask" limit on the bjdmk.com.cn page, section
  "实战集成".  With N_q queries against N_k keys the triangle is aligned to
  the last query and key (query i sees keys j <= i + N_k - N_q), which is the
  same mask when N_q = N_k and makes N_q new queries against an N_k-key
  history the last N_q rows of the square problem.  A query that sees no key
  gets O = 0 and LSE = -inf (the logsumexp of an empty set).
* Partial results over disjoint key sets combine exactly through the LSE:
  ``LSE = ln sum_r exp(LSE_r)``, ``O = sum_r exp(LSE_r - LSE) O_r`` -- the
  logsumexp statistic the walkthrough keeps (section 3.1) is what makes
  such a merge possible.
* ``LSE_i = m_i + ln(l_i)``, the per-row logsumexp of the scaled scores, which
  is the one statistic FlashAttention-2 keeps for the backward pass
  (hotelren.com walkthrough, section 3.1).
* Backward: the exact gradients of the forward definition, which the fused
  backward reproduces by recomputation (bjdmk.com.cn "性能引擎"; pwwt.cn
  section "3. 重计算").  Five products, as the walkthrough's section 3.3
  counts them:  dV = P^T dO,  dP = dO V^T,  dS = P o (dP - rowsum(P o dP)),
  dQ = scale dS K,  dK = scale dS^T Q.

The oracle materialises S and P (one head at a time).  Query rows are taken
in chunks only to bound host memory at long sequence lengths: every row of S
and P is still formed in full, and dK / dV are the sums over all rows of the
per-row contributions.  There is no online softmax, no exp2 and no tiling of
the key dimension.
"""

from __future__ import annotations

import numpy as np

DEFAULT_ROW_CHUNK = 2048


def _f64(x) -> np.ndarray:
    """Exact upcast of a numpy array or torch tensor (fp16/bf16/fp32) to fp64."""
    if hasattr(x, "detach"):  # a torch tensor; bf16 has no numpy type
        import torch
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def default_scale(D: int) -> float:
    """1/sqrt(d_k) of the attention formula."""
    return 1.0 / np.sqrt(D)


def _head_rows(Q, K, V, rows, causal, scale, dO=None, offset=0):
    """Softmax attention for the query rows ``rows`` of one (batch, head).

    Q: [R, D] (the query vectors of ``rows``), K, V: [Nk, D], dO: [R, D].
    ``offset`` = N_k - N_q: with ``causal`` query i sees keys j <= i + offset.
    Returns a dict with S, P, O, LSE and, when dO is given, dP, Dvec, dS,
    dQ (rows only) and the contributions of these rows to dK, dV.  Rows that
    see no key have P = 0, O = 0, LSE = -inf and zero gradients.
    """
    Nk = K.shape[0]
    S = scale * (Q @ K.T)                                  # [R, Nk]
    if causal:
        cols = np.arange(Nk)[None, :]
        S = np.where(cols > np.asarray(rows)[:, None] + offset, -np.inf, S)
    m = S.max(axis=1) if Nk else np.full(S.shape[0], -np.inf)
    empty = np.isneginf(m)                                 # no visible key
    m_safe = np.where(empty, 0.0, m)                       # running max is not
    E = np.exp(S - m_safe[:, None])                        # needed: whole row
    l = E.sum(axis=1)
    P = E / np.where(empty, 1.0, l)[:, None]
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    out = {"S": S, "P": P, "O": P @ V, "LSE": lse}
    if dO is not None:
        dP = dO @ V.T
        dvec_p = (P * dP).sum(axis=1)                      # rowsum(P o dP)
        dvec_o = (dO * out["O"]).sum(axis=1)               # rowsum(dO o O)
        # Both sums are bounded by |dO_i|_1 * max|V|; they must agree to
        # rounding (1e-12 relative to that bound).
        bound = np.abs(dO).sum(axis=1) * (np.abs(V).max() if V.size else 0.0)
        assert np.all(np.abs(dvec_p - dvec_o) <= 1e-12 * np.maximum(bound, 1e-300)), \
            "Dvec identity rowsum(P o dP) = rowsum(dO o O) violated"
        dS = P * (dP - dvec_p[:, None])
        out.update(dP=dP, Dvec=dvec_p, dS=dS,
                   dQ=scale * (dS @ K),
                   dK_part=scale * (dS.T @ Q),
                   dV_part=P.T @ dO)
    return out


def attention_forward(q, k, v, causal: bool = False, scale: float | None = None,
                      row_chunk: int = DEFAULT_ROW_CHUNK):
    """O [B,Nq,H,D] and LSE [B,H,Nq] (natural log) for q [B,Nq,H,D] and
    k, v [B,Nk,H,D]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, N, H, D = q.shape
    offset = k.shape[1] - N
    scale = default_scale(D) if scale is None else float(scale)
    O = np.zeros((B, N, H, D))
    LSE = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            K, V = k[b, :, h, :], v[b, :, h, :]
            for r0 in range(0, N, row_chunk):
                rows = np.arange(r0, min(N, r0 + row_chunk))
                res = _head_rows(q[b, rows, h, :], K, V, rows, causal, scale, offset=offset)
                O[b, rows, h, :] = res["O"]
                LSE[b, h, rows] = res["LSE"]
    return O, LSE


def merge_partials(O_parts, LSE_parts):
    """Exact combination of attention results over disjoint key sets.

    O_parts: [P, B, N, H, D], LSE_parts: [P, B, H, N] (natural log; -inf for
    a part in which a row sees no key).  Returns O [B,N,H,D], LSE [B,H,N]:
    LSE = ln sum_r exp(LSE_r) and O = sum_r exp(LSE_r - LSE) O_r, with O = 0
    and LSE = -inf for rows no part covers.
    """
    O_parts, LSE_parts = _f64(O_parts), _f64(LSE_parts)
    m = LSE_parts.max(axis=0)                              # [B, H, N]
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(LSE_parts - m_safe[None])                   # [P, B, H, N]
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        LSE = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, tot)))
    wn = w / np.where(empty, 1.0, tot)[None]               # weights exp(LSE_r - LSE)
    O = np.einsum("pbhn,pbnhd->bnhd", wn, O_parts)
    return O, LSE


def attention_backward(q, k, v, dout, causal: bool = False,
                       scale: float | None = None,
                       row_chunk: int = DEFAULT_ROW_CHUNK, heads=None):
    """dQ [B,Nq,H,D], dK, dV [B,Nk,H,D] (fp64) of  L = sum(O o dout).

    ``heads``: optional list of (b, h) pairs to evaluate; the others are left
    zero (used where a full-size check covers only some heads).
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, N, H, D = q.shape
    offset = k.shape[1] - N
    scale = default_scale(D) if scale is None else float(scale)
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in pairs:
        K, V = k[b, :, h, :], v[b, :, h, :]
        for r0 in range(0, N, row_chunk):
            rows = np.arange(r0, min(N, r0 + row_chunk))
            res = _head_rows(q[b, rows, h, :], K, V, rows, causal, scale,
                             dO=dout[b, rows, h, :], offset=offset)
            dQ[b, rows, h, :] = res["dQ"]
            dK[b, :, h, :] += res["dK_part"]
            dV[b, :, h, :] += res["dV_part"]
    return dQ, dK, dV


def attention_rows(q, k, v, dout, b: int, h: int, rows, causal: bool = False,
                   scale: float | None = None):
    """O, LSE, Dvec and dQ at selected query rows of one (b, h).

    These quantities depend only on their own row of S and P, so a subset of
    rows is computed exactly without forming the other rows.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    D = q.shape[3]
    scale = default_scale(D) if scale is None else float(scale)
    rows = np.asarray(rows)
    dO = None if dout is None else _f64(dout)[b, rows, h, :]
    res = _head_rows(q[b, rows, h, :], k[b, :, h, :], v[b, :, h, :], rows,
                     causal, scale, dO=dO, offset=k.shape[1] - q.shape[1])
    keep = ("O", "LSE") if dO is None else ("O", "LSE", "Dvec", "dQ")
    return {key: res[key] for key in keep}


def attention_probs(q, k, causal: bool = False, scale: float | None = None):
    """The full probability matrix P [B,H,Nq,Nk] (small inputs only)."""
    q, k = _f64(q), _f64(k)
    B, N, H, D = q.shape
    Nk = k.shape[1]
    scale = default_scale(D) if scale is None else float(scale)
    P = np.zeros((B, H, N, Nk))
    zeros = np.zeros((Nk, D))
    for b in range(B):
        for h in range(H):
            P[b, h] = _head_rows(q[b, :, h, :], k[b, :, h, :], zeros,
                                 np.arange(N), causal, scale, offset=Nk - N)["P"]
    return P


def row_dvec(o, dout):
    """Dvec [B,H,N] = rowsum(dO o O), the backward preprocess quantity."""
    o, dout = _f64(o), _f64(dout)
    return np.einsum("bnhd,bnhd->bhn", o, dout)

"""Pins for the CPU fp64 oracle: checks against what the pages and the
mathematics fix, independent of the oracle's own code path.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
its pin.  The tests run every pin on the oracle as written, and
``test_mutants_are_caught`` plants plausible mistakes into a copy of the
oracle's core (a dropped term, a wrong sign, a transposed operand, an
off-by-one mask) and checks that at least one pin fails for each.
"""

import inspect
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

from oracle import attention as oa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example_d1.json")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _qkv(B, N, H, D, seed):
    return (_rand((B, N, H, D), seed), _rand((B, N, H, D), seed + 1),
            _rand((B, N, H, D), seed + 2), _rand((B, N, H, D), seed + 3))


# ---------------------------------------------------------------- pins

def pin_rows_sum_to_one():
    """P1: every row of P is a probability vector (definition of softmax)."""
    q, k, _, _ = _qkv(2, 19, 3, 8, 11)
    for causal in (False, True):
        P = oa.attention_probs(q, k, causal=causal)
        assert np.all(P >= 0)
        assert np.max(np.abs(P.sum(axis=-1) - 1.0)) <= 1e-12
        if causal:
            assert np.all(np.triu(P[0, 0], 1) == 0.0)


def pin_constant_key():
    """P2: identical keys give uniform attention: O = mean(V) (running mean
    when causal), LSE = scale q.k + ln(#visible), and dQ = 0."""
    B, N, H, D = 1, 13, 2, 5
    q, _, v, do = _qkv(B, N, H, D, 21)
    kvec = _rand((1, 1, H, D), 25)
    k = np.broadcast_to(kvec, (B, N, H, D)).copy()
    scale = 0.37
    for causal in (False, True):
        O, LSE = oa.attention_forward(q, k, v, causal=causal, scale=scale)
        dQ, _, _ = oa.attention_backward(q, k, v, do, causal=causal, scale=scale)
        cnt = np.arange(1, N + 1) if causal else np.full(N, N)
        for h in range(H):
            if causal:
                mean = np.cumsum(v[0, :, h], axis=0) / cnt[:, None]
            else:
                mean = np.broadcast_to(v[0, :, h].mean(axis=0), (N, D))
            assert np.max(np.abs(O[0, :, h] - mean)) <= 1e-12
            lse = scale * q[0, :, h] @ kvec[0, 0, h] + np.log(cnt)
            assert np.max(np.abs(LSE[0, h] - lse)) <= 1e-12
        assert np.max(np.abs(dQ)) <= 1e-12


def pin_causal_rows():
    """P3: causal row 0 is V[0] with LSE = scale q0.k0; the last causal row is
    the last non-causal row; rows j > i of K/V do not affect causal row i."""
    B, N, H, D = 2, 11, 2, 6
    q, k, v, _ = _qkv(B, N, H, D, 31)
    scale = 0.5
    O, LSE = oa.attention_forward(q, k, v, causal=True, scale=scale)
    On, LSEn = oa.attention_forward(q, k, v, causal=False, scale=scale)
    assert np.max(np.abs(O[:, 0] - v[:, 0])) <= 1e-15
    lse0 = scale * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0])
    assert np.max(np.abs(LSE[:, :, 0] - lse0)) <= 1e-14
    assert np.max(np.abs(O[:, -1] - On[:, -1])) <= 1e-12
    assert np.max(np.abs(LSE[:, :, -1] - LSEn[:, :, -1])) <= 1e-12
    i = 4
    k2, v2 = k.copy(), v.copy()
    k2[:, i + 1:] = _rand(k2[:, i + 1:].shape, 35)
    v2[:, i + 1:] = _rand(v2[:, i + 1:].shape, 36)
    O2, LSE2 = oa.attention_forward(q, k2, v2, causal=True, scale=scale)
    assert np.array_equal(O2[:, : i + 1], O[:, : i + 1])
    assert np.array_equal(LSE2[:, :, : i + 1], LSE[:, :, : i + 1])


def pin_closed_forms():
    """P4: scale = 0 is uniform attention (dQ = dK = 0, dV_j = sum_i dO_i/#i);
    constant V gives O = v and dQ = dK = 0; N = 1 gives O = V, LSE = s q.k."""
    B, N, H, D = 1, 9, 2, 4
    q, k, v, do = _qkv(B, N, H, D, 41)
    for causal in (False, True):
        O, LSE = oa.attention_forward(q, k, v, causal=causal, scale=0.0)
        dQ, dK, dV = oa.attention_backward(q, k, v, do, causal=causal, scale=0.0)
        cnt = np.arange(1, N + 1) if causal else np.full(N, N)
        assert np.max(np.abs(LSE - np.log(cnt)[None, None, :])) <= 1e-14
        assert np.max(np.abs(dQ)) <= 1e-14 and np.max(np.abs(dK)) <= 1e-14
        w = do / cnt[None, :, None, None]                 # dO_i / #visible(i)
        if causal:                                        # dV_j = sum_{i>=j}
            expect = np.flip(np.cumsum(np.flip(w, 1), axis=1), 1)
        else:
            expect = np.broadcast_to(w.sum(axis=1, keepdims=True), w.shape)
        assert np.max(np.abs(dV - expect)) <= 1e-12
    vconst = np.broadcast_to(_rand((1, 1, H, D), 45), (B, N, H, D)).copy()
    for causal in (False, True):
        O, _ = oa.attention_forward(q, k, vconst, causal=causal)
        dQ, dK, _ = oa.attention_backward(q, k, vconst, do, causal=causal)
        assert np.max(np.abs(O - vconst)) <= 1e-12
        assert np.max(np.abs(dQ)) <= 1e-12 and np.max(np.abs(dK)) <= 1e-12
    q1, k1, v1, _ = _qkv(3, 1, 2, 7, 47)
    O, LSE = oa.attention_forward(q1, k1, v1, scale=0.3)
    assert np.array_equal(O, v1)
    assert np.max(np.abs(LSE - 0.3 * np.einsum("bnhd,bnhd->bhn", q1, k1))) <= 1e-14


def pin_gradient_sums():
    """P5: sum_j dK_j = 0 (each row of dS sums to zero);  P6: sum_j dV_j =
    sum_i dO_i (each row of P sums to one)."""
    q, k, v, do = _qkv(2, 17, 3, 8, 51)
    for causal in (False, True):
        _, dK, dV = oa.attention_backward(q, k, v, do, causal=causal)
        assert np.max(np.abs(dK.sum(axis=1))) <= 1e-12
        assert np.max(np.abs(dV.sum(axis=1) - do.sum(axis=1))) <= 1e-12


def pin_permutations():
    """P7: permuting K and V rows together leaves O unchanged (non-causal);
    permuting Q rows permutes O and LSE."""
    q, k, v, _ = _qkv(1, 15, 2, 6, 61)
    O, LSE = oa.attention_forward(q, k, v)
    perm = np.random.default_rng(62).permutation(15)
    O2, LSE2 = oa.attention_forward(q, k[:, perm], v[:, perm])
    assert np.max(np.abs(O2 - O)) <= 1e-12 and np.max(np.abs(LSE2 - LSE)) <= 1e-12
    O3, LSE3 = oa.attention_forward(q[:, perm], k, v)
    assert np.max(np.abs(O3 - O[:, perm])) <= 1e-12
    assert np.max(np.abs(LSE3 - LSE[:, :, perm])) <= 1e-12


def pin_dvec_identity():
    """P8: rowsum(dO o O) equals rowsum(P o dP) (the preprocess quantity)."""
    q, k, v, do = _qkv(1, 12, 2, 5, 71)
    O, _ = oa.attention_forward(q, k, v, causal=True)
    dvec = oa.row_dvec(O, do)
    for h in range(2):
        r = oa.attention_rows(q, k, v, do, 0, h, np.arange(12), causal=True)
        assert np.max(np.abs(r["Dvec"] - dvec[0, h])) <= 1e-12


def _loss(q, k, v, do, causal, scale):
    O, _ = oa.attention_forward(q, k, v, causal=causal, scale=scale)
    return float(np.sum(O * do))


FD_SHAPES = [(1, 1, 1, 1), (1, 2, 1, 3), (1, 3, 1, 2), (2, 5, 3, 4), (1, 8, 1, 4)]


def pin_finite_differences(shapes=FD_SHAPES):
    """P9: analytic dQ, dK, dV equal central finite differences (fp64,
    h = 1e-6) of L = sum(O o dO) to 1e-6 relative."""
    h = 1e-6
    for (B, N, H, D) in shapes:
        q, k, v, do = _qkv(B, N, H, D, 81 + N)
        for causal in (False, True):
            for scale in (1.0 / math.sqrt(D), 0.7):
                grads = oa.attention_backward(q, k, v, do, causal=causal, scale=scale)
                args = [q, k, v]
                for which in range(3):
                    fd = np.zeros_like(args[which])
                    for idx in np.ndindex(*args[which].shape):
                        plus = [a.copy() for a in args]
                        minus = [a.copy() for a in args]
                        plus[which][idx] += h
                        minus[which][idx] -= h
                        fd[idx] = (_loss(*plus, do, causal, scale)
                                   - _loss(*minus, do, causal, scale)) / (2 * h)
                    an = grads[which]
                    err = np.max(np.abs(fd - an))
                    assert err <= 1e-6 * max(1.0, np.max(np.abs(an))), \
                        (B, N, H, D, causal, scale, which, err)


def pin_library_routines():
    """P10: torch's CPU fp64 scaled_dot_product_attention (and its autograd
    gradients) and scipy's logsumexp agree with the oracle to 1e-12."""
    B, N, H, D = 2, 23, 3, 16
    q, k, v, do = _qkv(B, N, H, D, 91)
    for causal in (False, True):
        for scale in (None, 0.7):
            O, LSE = oa.attention_forward(q, k, v, causal=causal, scale=scale)
            dQ, dK, dV = oa.attention_backward(q, k, v, do, causal=causal, scale=scale)
            tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3), requires_grad=True)
                          for x in (q, k, v))
            out = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                 scale=scale)
            out.backward(torch.tensor(do.transpose(0, 2, 1, 3)))
            ref = out.detach().numpy().transpose(0, 2, 1, 3)
            assert np.max(np.abs(O - ref)) <= 1e-12
            for mine, t in ((dQ, tq), (dK, tk), (dV, tv)):
                g = t.grad.numpy().transpose(0, 2, 1, 3)
                assert np.max(np.abs(mine - g)) <= 1e-12
            s = 1.0 / math.sqrt(D) if scale is None else scale
            for b in range(B):
                for h in range(H):
                    logits = s * q[b, :, h] @ k[b, :, h].T
                    if causal:
                        logits[np.triu_indices(N, 1)] = -np.inf
                    lse = scipy.special.logsumexp(logits, axis=1)
                    assert np.max(np.abs(LSE[b, h] - lse)) <= 1e-12


def pin_worked_example():
    """P11: the hand-derived D = 1 example (tests/golden/worked_example_d1.json)."""
    with open(GOLDEN) as f:
        g = json.load(f)
    inp = g["inputs"]
    shape = (1, 2, 1, 1)
    q, k, v, do = (np.array(inp[n], dtype=np.float64).reshape(shape)
                   for n in ("q", "k", "v", "do"))
    for key, causal in (("noncausal", False), ("causal", True)):
        exp = g[key]
        O, LSE = oa.attention_forward(q, k, v, causal=causal, scale=inp["scale"])
        dQ, dK, dV = oa.attention_backward(q, k, v, do, causal=causal,
                                           scale=inp["scale"])
        for name, got in (("O", O), ("LSE", LSE), ("dQ", dQ), ("dK", dK), ("dV", dV)):
            assert np.max(np.abs(got.ravel() - np.array(exp[name]))) <= 1e-12, \
                (key, name, got.ravel(), exp[name])


def pin_sampled_rows_match_full():
    """attention_rows at a subset of rows equals the full computation."""
    q, k, v, do = _qkv(1, 40, 2, 8, 101)
    for causal in (False, True):
        O, LSE = oa.attention_forward(q, k, v, causal=causal)
        dQ, _, _ = oa.attention_backward(q, k, v, do, causal=causal)
        rows = [0, 3, 17, 39]
        r = oa.attention_rows(q, k, v, do, 0, 1, rows, causal=causal)
        assert np.max(np.abs(r["O"] - O[0, rows, 1])) <= 1e-14
        assert np.max(np.abs(r["LSE"] - LSE[0, 1, rows])) <= 1e-14
        assert np.max(np.abs(r["dQ"] - dQ[0, rows, 1])) <= 1e-14
        # row chunking bounds memory only: results do not depend on it
        O2, LSE2 = oa.attention_forward(q, k, v, causal=causal, row_chunk=7)
        g2 = oa.attention_backward(q, k, v, do, causal=causal, row_chunk=7)
        assert np.max(np.abs(O2 - O)) <= 1e-14
        assert np.max(np.abs(g2[0] - dQ)) <= 1e-14


def _close(a, b, tol=1e-12):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, (a.shape, b.shape)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin) and np.array_equal(a[~fin], b[~fin])
    assert np.max(np.abs(a[fin] - b[fin]), initial=0.0) <= tol * max(1.0, np.max(np.abs(b[fin]), initial=0.0))


def pin_offset_causal_matches_square():
    """P12: N_q < N_k queries under the causal mask aligned to the last key
    see exactly what the last N_q rows of the square causal problem see:
    square problem = queries [prefix; q] against the same keys, with dO = 0
    on the prefix rows (so they add nothing to dK, dV).  The last query
    sees every key, as without the mask."""
    B, Nq, Nk, H, D = 2, 5, 12, 2, 4
    q, do = _rand((B, Nq, H, D), 121), _rand((B, Nq, H, D), 124)
    k, v = _rand((B, Nk, H, D), 122), _rand((B, Nk, H, D), 123)
    prefix = _rand((B, Nk - Nq, H, D), 125)
    qs = np.concatenate([prefix, q], axis=1)
    dos = np.concatenate([np.zeros_like(prefix), do], axis=1)
    for scale in (None, 0.6):
        O, LSE = oa.attention_forward(q, k, v, causal=True, scale=scale)
        Os, LSEs = oa.attention_forward(qs, k, v, causal=True, scale=scale)
        _close(O, Os[:, Nk - Nq:])
        _close(LSE, LSEs[:, :, Nk - Nq:])
        dQ, dK, dV = oa.attention_backward(q, k, v, do, causal=True, scale=scale)
        dQs, dKs, dVs = oa.attention_backward(qs, k, v, dos, causal=True, scale=scale)
        _close(dQ, dQs[:, Nk - Nq:])
        _close(dK, dKs)
        _close(dV, dVs)
        On, LSEn = oa.attention_forward(q, k, v, causal=False, scale=scale)
        _close(O[:, -1], On[:, -1])
        _close(LSE[:, :, -1], LSEn[:, :, -1])


def pin_offset_more_queries_than_keys():
    """P13: with N_q > N_k and the same alignment, the first N_q - N_k
    queries see no key (O = 0, LSE = -inf, dQ = 0) and the rest are the
    square causal problem on the last N_k queries."""
    B, Nq, Nk, H, D = 1, 9, 4, 2, 3
    q, do = _rand((B, Nq, H, D), 131), _rand((B, Nq, H, D), 134)
    k, v = _rand((B, Nk, H, D), 132), _rand((B, Nk, H, D), 133)
    O, LSE = oa.attention_forward(q, k, v, causal=True)
    dQ, dK, dV = oa.attention_backward(q, k, v, do, causal=True)
    cut = Nq - Nk
    assert np.all(O[:, :cut] == 0.0) and np.all(np.isneginf(LSE[:, :, :cut]))
    assert np.all(dQ[:, :cut] == 0.0)
    Os, LSEs = oa.attention_forward(q[:, cut:], k, v, causal=True)
    dQs, dKs, dVs = oa.attention_backward(q[:, cut:], k, v, do[:, cut:], causal=True)
    _close(O[:, cut:], Os)
    _close(LSE[:, :, cut:], LSEs)
    _close(dQ[:, cut:], dQs)
    _close(dK, dKs)
    _close(dV, dVs)


def pin_merge_partials():
    """P14: attention over a key set split into chunks, merged through the
    LSE, equals attention over the whole set: non-causal with three chunks;
    causal (N_k > N_q) as a non-causal part over the keys every query sees
    plus the causal part over the rest; a part in which no row sees a key
    changes nothing.  The merged LSE matches scipy's logsumexp of the parts."""
    B, Nq, Nk, H, D = 2, 6, 11, 2, 5
    q = _rand((B, Nq, H, D), 141)
    k, v = _rand((B, Nk, H, D), 142), _rand((B, Nk, H, D), 143)
    O, LSE = oa.attention_forward(q, k, v)
    cuts = [0, 4, 8, Nk]
    parts = [oa.attention_forward(q, k[:, a:b], v[:, a:b]) for a, b in zip(cuts, cuts[1:])]
    Op = np.stack([p[0] for p in parts])
    Lp = np.stack([p[1] for p in parts])
    Om, Lm = oa.merge_partials(Op, Lp)
    _close(Om, O)
    _close(Lm, LSE)
    _close(Lm, scipy.special.logsumexp(Lp, axis=0))
    # a part that covers no key for any row
    Om2, Lm2 = oa.merge_partials(np.concatenate([Op, np.zeros_like(Op[:1])]),
                                 np.concatenate([Lp, np.full_like(Lp[:1], -np.inf)]))
    _close(Om2, O)
    _close(Lm2, LSE)
    # causal, N_k > N_q: keys [0, s) with s <= N_k - N_q + 1 are seen by every query
    s = Nk - Nq + 1
    Oc, LSEc = oa.attention_forward(q, k, v, causal=True)
    p0 = oa.attention_forward(q, k[:, :s], v[:, :s], causal=False)
    p1 = oa.attention_forward(q, k[:, s:], v[:, s:], causal=True)
    Omc, Lmc = oa.merge_partials(np.stack([p0[0], p1[0]]), np.stack([p0[1], p1[1]]))
    _close(Omc, Oc)
    _close(Lmc, LSEc)


ALL_PINS = [pin_rows_sum_to_one, pin_constant_key, pin_causal_rows, pin_closed_forms,
            pin_gradient_sums, pin_permutations, pin_dvec_identity,
            pin_finite_differences, pin_library_routines, pin_worked_example,
            pin_sampled_rows_match_full, pin_offset_causal_matches_square,
            pin_offset_more_queries_than_keys, pin_merge_partials]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()


def test_bf16_inputs_upcast_exactly():
    """Half-precision torch tensors reach the oracle bit-exactly in fp64."""
    t = torch.randn(1, 5, 1, 3).to(torch.bfloat16)
    a = oa._f64(t)
    assert a.dtype == np.float64
    assert np.array_equal(a, t.float().numpy().astype(np.float64))


# ------------------------------------------------------- planted mistakes

MUTANTS = {
    "dropped_scale_in_S": ("S = scale * (Q @ K.T)", "S = (Q @ K.T)"),
    "mask_includes_diagonal": ("cols > np.asarray(rows)", "cols >= np.asarray(rows)"),
    "mask_wrong_triangle": ("cols > np.asarray(rows)", "cols < np.asarray(rows)"),
    "lse_without_max": ("m_safe + np.log(np.where(empty, 1.0, l))",
                        "np.log(np.where(empty, 1.0, l))"),
    "lse_log2": ("m_safe + np.log(np.where(empty, 1.0, l))",
                 "m_safe + np.log2(np.where(empty, 1.0, l))"),
    "no_max_shift_in_lse": ("E = np.exp(S - m_safe[:, None])", "E = np.exp(S)"),
    "normaliser_transposed": ("P = E / np.where(empty, 1.0, l)[:, None]",
                              "P = E / np.where(empty, 1.0, l)[None, :]"),
    "offset_ignored": ("[:, None] + offset, -np.inf", "[:, None], -np.inf"),
    "offset_sign": ("[:, None] + offset, -np.inf", "[:, None] - offset, -np.inf"),
    "output_transposed": ('"O": P @ V', '"O": P.T @ V'),
    "dP_uses_K": ("dP = dO @ V.T", "dP = dO @ K.T"),
    "dS_sign": ("dS = P * (dP - dvec_p[:, None])", "dS = P * (dvec_p[:, None] - dP)"),
    "dS_drops_dvec": ("dS = P * (dP - dvec_p[:, None])", "dS = P * dP"),
    "dQ_without_scale": ("dQ=scale * (dS @ K)", "dQ=(dS @ K)"),
    "dQ_uses_V": ("dQ=scale * (dS @ K)", "dQ=scale * (dS @ V)"),
    "dK_uses_dO": ("dK_part=scale * (dS.T @ Q)", "dK_part=scale * (dS.T @ dO)"),
    "dK_without_scale": ("dK_part=scale * (dS.T @ Q)", "dK_part=(dS.T @ Q)"),
    "dV_transposed": ("dV_part=P.T @ dO", "dV_part=P @ dO"),
    "dV_uses_dS": ("dV_part=P.T @ dO", "dV_part=dS.T @ dO"),
}

# Cheap subset of the pins used against each mutant (the full FD sweep is
# slow; two small shapes cover every term).
QUICK_PINS = [pin_worked_example, pin_rows_sum_to_one, pin_constant_key,
              pin_causal_rows, pin_gradient_sums, pin_library_routines,
              pin_offset_causal_matches_square, pin_offset_more_queries_than_keys,
              lambda: pin_finite_differences([(1, 3, 1, 2), (2, 5, 3, 4)])]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(name, monkeypatch):
    old, new = MUTANTS[name]
    src = inspect.getsource(oa._head_rows)
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    ns = dict(vars(oa))
    exec(src.replace(old, new), ns)
    monkeypatch.setattr(oa, "_head_rows", ns["_head_rows"])
    caught = []
    for pin in QUICK_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, FloatingPointError, RuntimeError):
            caught.append(getattr(pin, "__name__", "fd"))
    assert caught, f"mutant {name} passed every pin"


# Planted mistakes in the merge of partial results.
MERGE_MUTANTS = {
    "merge_lse_without_log": ("m_safe + np.log(np.where(empty, 1.0, tot))",
                              "m_safe + np.where(empty, 1.0, tot)"),
    "merge_weights_unnormalised": ("wn = w / np.where(empty, 1.0, tot)[None]", "wn = w"),
    "merge_first_part_only": ("w = np.exp(LSE_parts - m_safe[None])",
                              "w = np.exp(LSE_parts[:1] - m_safe[None])"),
    "merge_weights_without_exp": ("w = np.exp(LSE_parts - m_safe[None])",
                                  "w = LSE_parts - m_safe[None]"),
}


@pytest.mark.parametrize("name", sorted(MERGE_MUTANTS))
def test_merge_mutants_are_caught(name, monkeypatch):
    old, new = MERGE_MUTANTS[name]
    src = inspect.getsource(oa.merge_partials)
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    ns = dict(vars(oa))
    exec(src.replace(old, new), ns)
    monkeypatch.setattr(oa, "merge_partials", ns["merge_partials"])
    with pytest.raises((AssertionError, ValueError, FloatingPointError)):
        with np.errstate(all="ignore"):
            pin_merge_partials()

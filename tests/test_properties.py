"""GPU checks of the structural properties of exact attention, on inputs
built so that the exact result is known in closed form or must not change
(the definition: softmax of the scaled scores, lower-triangular mask for
causal; pwwt.cn page, sections on the attention formula and the causal
mask).  Each case spans several K/V tiles and a ragged tail.

  * Constant keys: every score of a row is equal, so O_i is the mean of
    the visible V rows, LSE_i = scale q_i.k + ln(#visible) and dQ = 0 (each
    row of dS sums to zero and meets the same k).
  * Causal prefix: row 0 sees key 0 only, so O_0 = V_0 and LSE_0 = scale
    q_0.k_0; changing K/V rows from t on leaves rows before t unchanged.
    The kernels keep this bit for bit when t is a multiple of 32 (the rows
    of one wave) and the change keeps the head's largest |K| and |V| (here:
    rows t.. reversed): masked keys enter only as exact zeros, but one wave
    moves the softmax reference point of all its rows together, and the
    fixed-point dQ unit follows those maxima.  Other t: within tolerance.
  * Constant values: O = v, and dQ = dK = 0 (dP - Dvec vanishes).
  * Permutations: permuting the query rows (with their dO rows) permutes O,
    LSE and dQ; permuting K and V rows together leaves O, LSE and dQ
    unchanged and permutes dK and dV.  Within the usual tolerances (the
    summation order and the reference-point updates differ).
"""

import sys

import numpy as np
import pytest
import torch

import io_aware_exact_02_amd as fa
from oracle import attention as oa
from workloads import random_qkv

pytestmark = pytest.mark.gpu

O_TOL = 1e-2
LSE_TOL = 1e-3
G_TOL = 5e-2
N = 333


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _run(q, k, v, do, causal, scale=None):
    dev = torch.device("cuda")
    q, k, v, do = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa.fwd(q, k, v, causal=causal, softmax_scale=scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    return {name: t.cpu() for name, t in zip(("O", "LSE", "dQ", "dK", "dV"), (o, lse, dq, dk, dv))}


def _f64(t):
    return t.to(torch.float64).numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_constant_keys(D, causal, dtype):
    what = f"constant keys D={D} causal={causal} {dtype}"
    _say("case", what)
    inp = random_qkv(1, N, 2, D, dtype, seed=7600 + D)
    k = inp["k"][:, :1].expand(-1, N, -1, -1).contiguous()
    got = _run(inp["q"], k, inp["v"], inp["do"], causal)
    q64, k64, v64 = _f64(inp["q"]), _f64(k), _f64(inp["v"])
    scale = D ** -0.5
    count = np.arange(1, N + 1, dtype=np.float64) if causal else np.full(N, float(N))
    # O_i: mean of the visible V rows, [B, N, H, D].
    if causal:
        O = np.cumsum(v64, axis=1) / count[None, :, None, None]
    else:
        O = np.broadcast_to(v64.mean(axis=1, keepdims=True), v64.shape)
    # LSE_i = scale q_i.k + ln(count), [B, H, N].
    s = scale * np.einsum("bnhd,bhd->bhn", q64, k64[:, 0])
    LSE = s + np.log(count)[None, None, :]
    eo = np.max(np.abs(_f64(got["O"]) - O))
    el = np.max(np.abs(_f64(got["LSE"]) - LSE))
    assert eo <= O_TOL, f"{what}: O {eo:.3e}"
    assert el <= LSE_TOL, f"{what}: LSE {el:.3e}"
    # dQ = 0 exactly in the mathematics; the kernel's dS is rounded to the
    # input type before the product, so the bar is the gradient tolerance
    # taken relative to dK, the other score gradient of the same problem.
    _, dK, dV = oa.attention_backward(inp["q"], k, inp["v"], inp["do"], causal=causal)
    dq_max = np.max(np.abs(_f64(got["dQ"])))
    assert dq_max <= G_TOL * np.max(np.abs(dK)), f"{what}: dQ {dq_max:.3e}"
    for name, ref in (("dK", dK), ("dV", dV)):
        err = np.max(np.abs(_f64(got[name]) - ref))
        assert err <= G_TOL * np.max(np.abs(ref)), f"{what}: {name} {err:.3e}"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
def test_causal_prefix(D, dtype):
    what = f"causal prefix D={D} {dtype}"
    _say("case", what)
    inp = random_qkv(1, N, 2, D, dtype, seed=7620 + D)
    got = _run(inp["q"], inp["k"], inp["v"], inp["do"], True)
    # Row 0: one visible key with weight exactly 1.
    assert torch.equal(got["O"][:, 0], inp["v"][:, 0]), f"{what}: O_0 != V_0"
    lse0 = (D ** -0.5) * np.einsum("bhd,bhd->bh", _f64(inp["q"][:, 0]), _f64(inp["k"][:, 0]))
    el = np.max(np.abs(_f64(got["LSE"][:, :, 0]) - lse0))
    assert el <= LSE_TOL, f"{what}: LSE_0 {el:.3e}"
    # Rows before t never see keys t.. : other K/V values there change nothing.
    for t in (32, 64, 192, 100):
        k2, v2 = inp["k"].clone(), inp["v"].clone()
        k2[:, t:] = inp["k"][:, t:].flip(1)
        v2[:, t:] = inp["v"][:, t:].flip(1)
        got2 = _run(inp["q"], k2, v2, inp["do"], True)
        if t % 32 == 0:
            assert torch.equal(got2["O"][:, :t], got["O"][:, :t]), f"{what}: O rows < {t} changed"
            assert torch.equal(got2["LSE"][:, :, :t], got["LSE"][:, :, :t]), f"{what}: LSE rows < {t}"
            assert torch.equal(got2["dQ"][:, :t], got["dQ"][:, :t]), f"{what}: dQ rows < {t} changed"
        else:
            eo = np.max(np.abs(_f64(got2["O"][:, :t]) - _f64(got["O"][:, :t])))
            el = np.max(np.abs(_f64(got2["LSE"][:, :, :t]) - _f64(got["LSE"][:, :, :t])))
            ref = _f64(got["dQ"][:, :t])
            eq = np.max(np.abs(_f64(got2["dQ"][:, :t]) - ref))
            assert eo <= O_TOL and el <= LSE_TOL, f"{what}: rows < {t}: O {eo:.3e} LSE {el:.3e}"
            assert eq <= G_TOL * np.max(np.abs(ref)), f"{what}: dQ rows < {t}: {eq:.3e}"


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_constant_values(D, causal):
    what = f"constant values D={D} causal={causal}"
    _say("case", what)
    inp = random_qkv(1, N, 2, D, "bf16", seed=7660 + D)
    v = inp["v"][:, :1].expand(-1, N, -1, -1).contiguous()
    got = _run(inp["q"], inp["k"], v, inp["do"], causal)
    # The weights sum to the normaliser, so O is v to within fp32 rounding,
    # far inside one bf16 step: the stored output is v itself.
    assert torch.equal(got["O"], v), f"{what}: O != v"
    # dQ = dK = 0: bar relative to dV, the nonzero gradient of the problem.
    _, _, dV = oa.attention_backward(inp["q"], inp["k"], v, inp["do"], causal=causal)
    bound = G_TOL * np.max(np.abs(dV))
    for name in ("dQ", "dK"):
        m = np.max(np.abs(_f64(got[name])))
        assert m <= bound, f"{what}: {name} {m:.3e} > {bound:.3e}"
    err = np.max(np.abs(_f64(got["dV"]) - dV))
    assert err <= bound, f"{what}: dV {err:.3e}"


@pytest.mark.parametrize("D", [64, 128])
def test_permutations(D):
    what = f"permutations D={D}"
    _say("case", what)
    inp = random_qkv(1, N, 2, D, "bf16", seed=7680 + D)
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
    base = _run(q, k, v, do, False)
    perm = torch.randperm(N, generator=torch.Generator("cpu").manual_seed(7690 + D))
    # Query rows (with their dO rows) permuted: outputs permuted alike.
    gq = _run(q[:, perm], k, v, do[:, perm], False)
    eo = np.max(np.abs(_f64(gq["O"]) - _f64(base["O"])[:, perm]))
    el = np.max(np.abs(_f64(gq["LSE"]) - _f64(base["LSE"])[:, :, perm]))
    assert eo <= O_TOL and el <= LSE_TOL, f"{what}: query permutation O {eo:.3e} LSE {el:.3e}"
    for name in ("dQ", "dK", "dV"):
        ref = _f64(base[name])[:, perm] if name == "dQ" else _f64(base[name])
        err = np.max(np.abs(_f64(gq[name]) - ref))
        assert err <= G_TOL * np.max(np.abs(ref)), f"{what}: query permutation {name} {err:.3e}"
    # Keys and values permuted together: a different summation order only.
    gk = _run(q, k[:, perm], v[:, perm], do, False)
    eo = np.max(np.abs(_f64(gk["O"]) - _f64(base["O"])))
    el = np.max(np.abs(_f64(gk["LSE"]) - _f64(base["LSE"])))
    assert eo <= O_TOL and el <= LSE_TOL, f"{what}: O {eo:.3e} LSE {el:.3e}"
    for name in ("dK", "dV"):
        ref = _f64(base[name])[:, perm]
        err = np.max(np.abs(_f64(gk[name]) - ref))
        assert err <= G_TOL * np.max(np.abs(ref)), f"{what}: {name} {err:.3e}"
    ref = _f64(base["dQ"])
    err = np.max(np.abs(_f64(gk["dQ"]) - ref))
    assert err <= G_TOL * np.max(np.abs(ref)), f"{what}: dQ {err:.3e}"

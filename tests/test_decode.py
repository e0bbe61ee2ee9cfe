"""GPU parity of the vector-unit forward that serves launches with at most
two query rows per (batch, head) -- one or two new tokens against a key
history -- through fa.fwd (unsplit: the kernel writes O and LSE itself;
split: fp32 partials merged by the split merge), against the fp64 oracle.

The kernel keeps the weights in fp32 (no matrix product, so no rounding of
P to the input type), so the O error is the output rounding plus fp32 sums:
the parity bar of the other forwards (O max-abs <= 1e-2, LSE max-abs <=
1e-3) holds with a wide margin, and rows that see no key give exactly
O = 0, LSE = -inf.  The score of a key is a sum over D/8 lanes that every
one of them holds bit for bit, and all combines run in a fixed order, so
repeated runs agree bitwise.
"""

import sys

import numpy as np
import pytest
import torch

import io_aware_exact_02_amd as fa
from io_aware_exact_02_amd import _lib
from oracle import attention as oa
from workloads import random_qkv

pytestmark = pytest.mark.gpu

O_TOL = 1e-2
LSE_TOL = 1e-3
G_TOL = 5e-2


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _inputs(B, Nq, Nk, H, D, dtype, seed):
    a = random_qkv(B, Nq, H, D, dtype, seed)
    b = random_qkv(B, Nk, H, D, dtype, seed + 1)
    return {"q": a["q"], "do": a["do"], "k": b["k"], "v": b["v"]}


def _check(o, lse, O, LSE, what):
    empty = np.isneginf(LSE)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: empty rows differ"
    if empty.any():
        assert np.all(o[np.transpose(empty, (0, 2, 1))] == 0.0), f"{what}: empty rows not 0"
    assert np.all(np.isfinite(o)), what
    eo = np.max(np.abs(o - O))
    assert eo <= O_TOL, f"{what}: O max-abs {eo:.3e}"
    if (~empty).any():
        el = np.max(np.abs(lse[~empty] - LSE[~empty]))
        assert el <= LSE_TOL, f"{what}: LSE max-abs {el:.3e}"


# (B, H, Nq, Nk, D, causal, dtype, num_splits; None = fa_fwd_split_count's
# choice).  Key counts below, at and past the kernel's chunks (256 keys per
# workgroup pass at head_dim 64, 128 at 128), ragged last splits, a split
# of one key, Nq > Nk (causal: row 0 sees no key), more splits than
# 128-key ranges.
CASES = [
    (2, 3, 1, 1, 64, True, "bf16", 1),
    (2, 3, 2, 1, 64, True, "bf16", 1),      # row 0 sees no key
    (2, 3, 2, 1, 128, False, "f16", 1),
    (1, 4, 1, 7, 128, True, "f16", 1),
    (1, 4, 2, 255, 64, True, "bf16", 1),
    (1, 4, 2, 257, 64, False, "f16", 1),
    (1, 4, 1, 129, 64, True, "bf16", 2),    # second split: one key
    (1, 4, 2, 129, 128, True, "bf16", 2),   # ... which row 0 cannot see
    (2, 2, 1, 1000, 64, False, "f16", 5),
    (2, 2, 2, 1000, 128, True, "bf16", 3),
    (1, 3, 1, 4097, 64, True, "bf16", None),
    (1, 3, 2, 4097, 128, False, "f16", None),
    (1, 2, 1, 300, 64, True, "bf16", 256),  # 256 requested, 3 ranges hold keys
    (3, 5, 2, 2500, 64, True, "f16", 7),
    (1, 2, 1, 20000, 128, True, "bf16", 64),
]


@pytest.mark.parametrize("B,H,Nq,Nk,D,causal,dtype,S", CASES)
def test_decode_parity(B, H, Nq, Nk, D, causal, dtype, S):
    what = f"decode B={B} H={H} Nq={Nq} Nk={Nk} D={D} causal={causal} {dtype} S={S}"
    _say("case", what)
    inp = _inputs(B, Nq, Nk, H, D, dtype, 9900 + Nq + 7 * Nk + D)
    dev = torch.device("cuda")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, causal=causal, num_splits=S)
    torch.cuda.synchronize()
    O, LSE = oa.attention_forward(inp["q"], inp["k"], inp["v"], causal=causal)
    _check(_f64(o), _f64(lse), O, LSE, what)


def test_decode_long_history_all_heads():
    """One new token per head against 16K keys, 16 heads, the automatic
    split count, every head against the oracle."""
    _say("case decode B1 H16 Nk16384")
    assert _lib.load().fa_fwd_split_count(1, 16, 1, 16384, 64, 1) > 1
    inp = _inputs(1, 1, 16384, 16, 64, "bf16", 9950)
    dev = torch.device("cuda")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    O, LSE = oa.attention_forward(inp["q"], inp["k"], inp["v"], causal=True)
    _check(_f64(o), _f64(lse), O, LSE, "decode 16K")


@pytest.mark.parametrize("scale", [-0.3, 0.0, 2.0])
def test_decode_scale(scale):
    """A negative scale (scores enter with the opposite sign), zero (uniform
    weights: O is the mean of the visible V rows) and a sharp one."""
    what = f"decode scale={scale}"
    _say("case", what)
    inp = _inputs(1, 2, 700, 3, 64, "bf16", 9960)
    dev = torch.device("cuda")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    for S in (1, 3):
        o, lse = fa.fwd(q, k, v, causal=True, softmax_scale=scale, num_splits=S)
        torch.cuda.synchronize()
        O, LSE = oa.attention_forward(inp["q"], inp["k"], inp["v"], causal=True, scale=scale)
        _check(_f64(o), _f64(lse), O, LSE, f"{what} S={S}")
    if scale == 0.0:
        vv = _f64(inp["v"])
        mean = np.stack([vv[:, :699].mean(axis=1), vv.mean(axis=1)], axis=1)  # rows see 699, 700
        assert np.max(np.abs(_f64(o) - mean)) <= O_TOL


def test_decode_strided_views():
    """K and V as views of one packed [B, N, 2, H, D] tensor (n-stride 2*H*D),
    q a view with a wider n-stride, O written into a view of a wider tensor."""
    _say("case decode strided")
    B, Nq, Nk, H, D = 2, 2, 900, 3, 128
    inp = _inputs(B, Nq, Nk, H, D, "f16", 9970)
    dev = torch.device("cuda")
    kv = torch.stack([inp["k"], inp["v"]], dim=2).to(dev)
    k, v = kv.unbind(dim=2)
    qw = torch.zeros((B, Nq, H, 2 * D), dtype=torch.float16, device=dev)
    qw[..., :D] = inp["q"].to(dev)
    q = qw[..., :D]
    wide = torch.full((B, Nq, H, 2 * D), float("nan"), dtype=torch.float16, device=dev)
    out = wide[..., D:]
    O, LSE = oa.attention_forward(inp["q"], inp["k"], inp["v"], causal=False)
    for S in (1, 4):
        o, lse = fa.fwd(q, k, v, causal=False, num_splits=S, out=out)
        torch.cuda.synchronize()
        assert o.data_ptr() == out.data_ptr()
        assert torch.isnan(wide[..., :D]).all(), "wrote outside the output view"
        _check(_f64(o), _f64(lse), O, LSE, f"decode strided S={S}")


def test_decode_bitwise_repeatable():
    _say("case decode repeat")
    inp = _inputs(2, 2, 3000, 4, 64, "bf16", 9980)
    dev = torch.device("cuda")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    runs = []
    for _ in range(3):
        o, lse = fa.fwd(q, k, v, causal=True, num_splits=6)
        torch.cuda.synchronize()
        runs.append((o.clone(), lse.clone()))
    for o, lse in runs[1:]:
        assert torch.equal(o, runs[0][0]) and torch.equal(lse, runs[0][1])


@pytest.mark.parametrize("D,causal", [(64, True), (128, False)])
def test_decode_then_backward(D, causal):
    """The backward recomputes P from this forward's LSE: gradients of one
    and two new rows against the oracle."""
    for Nq in (1, 2):
        what = f"decode fwd+bwd Nq={Nq} D={D} causal={causal}"
        _say("case", what)
        inp = _inputs(1, Nq, 1500, 3, D, "bf16", 9990 + D + Nq)
        dev = torch.device("cuda")
        q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
        o, lse = fa.fwd(q, k, v, causal=causal)
        dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal)
        torch.cuda.synchronize()
        O, LSE = oa.attention_forward(inp["q"], inp["k"], inp["v"], causal=causal)
        _check(_f64(o), _f64(lse), O, LSE, what)
        refs = oa.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], causal=causal)
        for name, got, ref in zip(("dQ", "dK", "dV"), (dq, dk, dv), refs):
            mag = np.max(np.abs(ref))
            err = np.max(np.abs(_f64(got) - ref))
            assert err <= G_TOL * mag, f"{what} {name} {err:.3e} > {G_TOL * mag:.3e}"


def test_three_rows_take_the_tiled_kernels():
    """Three rows per head go to the matrix-core forward; the result is the
    same function (oracle parity on both sides of the boundary)."""
    _say("case decode 2 vs 3 rows")
    inp = _inputs(1, 3, 1200, 2, 64, "bf16", 9995)
    dev = torch.device("cuda")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o3, lse3 = fa.fwd(q, k, v, causal=True)
    o2, lse2 = fa.fwd(q[:, 1:], k, v, causal=True)  # the last two rows alone
    torch.cuda.synchronize()
    O, LSE = oa.attention_forward(inp["q"], inp["k"], inp["v"], causal=True)
    _check(_f64(o3), _f64(lse3), O, LSE, "3 rows")
    _check(_f64(o2), _f64(lse2), O[:, 1:], LSE[:, :, 1:], "last 2 rows")


def test_decode_graph_replay_matches_eager():
    """The decode forward captured in a HIP graph, split (partials, then the
    merge) and unsplit: every replay, with stale outputs and eager work in
    between, equals the eager result bit for bit."""
    _say("case decode graph replay")
    dev = torch.device("cuda")
    a = _inputs(2, 2, 3000, 3, 128, "bf16", 9997)
    b = _inputs(3, 1, 2000, 4, 64, "f16", 9998)
    qa, ka, va = (a[n].to(dev) for n in ("q", "k", "v"))
    qb, kb, vb = (b[n].to(dev) for n in ("q", "k", "v"))
    oa_e, la_e = fa.fwd(qa, ka, va, causal=True, num_splits=6)
    ob_e, lb_e = fa.fwd(qb, kb, vb, causal=False, num_splits=1)
    torch.cuda.synchronize()
    oa_, la_ = torch.empty_like(oa_e), torch.empty_like(la_e)
    ob_, lb_ = torch.empty_like(ob_e), torch.empty_like(lb_e)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fa.fwd(qa, ka, va, causal=True, num_splits=6, out=oa_, lse=la_)
        fa.fwd(qb, kb, vb, causal=False, num_splits=1, out=ob_, lse=lb_)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fwd(qa, ka, va, causal=True, num_splits=6, out=oa_, lse=la_)
        fa.fwd(qb, kb, vb, causal=False, num_splits=1, out=ob_, lse=lb_)
    for rep in range(3):
        for t in (oa_, la_, ob_, lb_):
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(oa_, oa_e) and torch.equal(la_, la_e), f"split replay {rep}"
        assert torch.equal(ob_, ob_e) and torch.equal(lb_, lb_e), f"unsplit replay {rep}"
        _ = torch.cos(qa.float()).sum()
        torch.cuda.synchronize()

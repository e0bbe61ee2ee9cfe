"""GPU parity of the key-split forward (fa_fwd_split, reached through
fa.fwd(num_splits=...)) against the fp64 oracle, and its agreement with the
unsplit forward on the same inputs.

The split forward computes the same function: each workgroup sees one range
of keys, writes an fp32 partial (O_r, LSE_r), and a second kernel combines
the partials with the exact merge rule that storing the logsumexp allows
(hotelren.com FlashAttention-2 walkthrough, section 3.1).  Bars: the parity
bar of the unsplit forward (O max-abs <= 1e-2, LSE max-abs <= 1e-3; rows that
see no key exactly O = 0, LSE = -inf), and gradients through the split
forward's O and LSE at <= 5e-2 * max|reference|.

Against the unsplit forward on the same inputs: the LSE comes from fp32 sums
on both sides, so it agrees to 1e-5.  O does not agree to the last bit,
because P is rounded to the input type (relative error u = 2^-9 for bf16,
2^-12 for fp16) and each side normalises by different sums of rounded
weights: a split divides by its own sum, the unsplit kernel by the sum over
all keys.  Each side is within u * max|v - O| <= 2u max|v| of the exact
result before the output rounding (a convex combination of rows with
weights off by at most u relative), so the two differ by at most
4u max|v| + 2^-8 |O| (bf16; 2^-11 for fp16).
"""

import sys

import numpy as np
import pytest
import torch

import io_aware_exact_02_amd as fa
from oracle import attention as oa
from workloads import random_qkv, sample_rows

pytestmark = pytest.mark.gpu

O_TOL = 1e-2
LSE_TOL = 1e-3
G_TOL = 5e-2
EPS = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}  # one output ulp relative to |O|
U = {"bf16": 2.0 ** -9, "f16": 2.0 ** -12}    # rounding of P to the input type


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _inputs(B, Nq, Nk, H, D, dtype, seed):
    a = random_qkv(B, Nq, H, D, dtype, seed)
    b = random_qkv(B, Nk, H, D, dtype, seed + 1)
    return {"q": a["q"], "do": a["do"], "k": b["k"], "v": b["v"]}


def _check_against_oracle(o, lse, O, LSE, what):
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


def _check_against_unsplit(o, lse, o1, lse1, vmax, dtype, what):
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse1)), what
    fin = ~np.isneginf(lse1)
    if fin.any():
        assert np.max(np.abs(lse[fin] - lse1[fin])) <= 1e-5, f"{what}: LSE vs unsplit"
    bound = 4 * U[dtype] * vmax + 2 * EPS[dtype] * np.abs(o1)
    assert np.all(np.abs(o - o1) <= bound), f"{what}: O vs unsplit {np.max(np.abs(o - o1)):.3e}"


# (B, H, Nq, Nk, D, causal, dtype, num_splits).  Together they reach the
# forward kernel forms a split launch of this size takes (head_dim 64 with 4
# waves, the split key-group form of head_dim 128 causal-paired and
# non-causal, the plain head_dim-128 causal form), both forms of the merge
# (one wave per row up to 4096 rows, D/8 threads per row above), ranges a
# row cannot see, rows that see no key, a split count above the number of
# 128-key ranges, and ragged key tails.
CASES = [
    (1, 4, 1, 1000, 64, True, "bf16", 4),      # one new query against a history
    (1, 4, 1, 1000, 128, False, "f16", 7),
    (2, 3, 17, 2000, 64, True, "bf16", 16),    # a short chunk of a long context
    (2, 3, 130, 1300, 128, True, "bf16", 5),
    (1, 2, 300, 300, 64, True, "f16", 3),      # square causal: early rows see 1 range
    (1, 2, 300, 300, 128, True, "bf16", 2),
    (1, 2, 600, 200, 64, True, "bf16", 2),     # Nq > Nk: rows that see no key
    (1, 2, 600, 200, 128, True, "f16", 2),
    (1, 3, 1024, 1024, 128, True, "bf16", 3),  # split, paired head_dim-128 form
    (1, 2, 257, 4096, 64, False, "bf16", 64),  # many splits
    (1, 2, 64, 129, 64, False, "f16", 256),    # more splits than 128-key ranges
    (2, 2, 1000, 3000, 128, False, "bf16", 3),
    (2, 4, 600, 1800, 64, True, "bf16", 3),    # 4800 rows: the per-thread merge
]


@pytest.mark.parametrize("B,H,Nq,Nk,D,causal,dtype,S", CASES)
def test_split_forward_parity(B, H, Nq, Nk, D, causal, dtype, S):
    what = f"split B={B} H={H} Nq={Nq} Nk={Nk} D={D} causal={causal} {dtype} S={S}"
    _say("case", what)
    inp = _inputs(B, Nq, Nk, H, D, dtype, 9100 + Nq + 3 * Nk + D + S)
    dev = torch.device("cuda")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, causal=causal, num_splits=S)
    o1, lse1 = fa.fwd(q, k, v, causal=causal, num_splits=1)
    torch.cuda.synchronize()
    O, LSE = oa.attention_forward(inp["q"], inp["k"], inp["v"], causal=causal)
    _check_against_oracle(_f64(o), _f64(lse), O, LSE, what)
    vmax = float(np.max(np.abs(_f64(inp["v"]))))
    _check_against_unsplit(_f64(o), _f64(lse), _f64(o1), _f64(lse1), vmax, dtype, what)


@pytest.mark.parametrize("D,causal", [(64, True), (128, False)])
def test_split_forward_then_backward(D, causal):
    """The backward recomputes P from the split forward's LSE: gradients of a
    decoding-like shape against the oracle."""
    what = f"split fwd+bwd D={D} causal={causal}"
    _say("case", what)
    inp = _inputs(1, 40, 1500, 3, D, "bf16", 9300 + D)
    dev = torch.device("cuda")
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=causal, num_splits=6)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal)
    torch.cuda.synchronize()
    O, LSE = oa.attention_forward(inp["q"], inp["k"], inp["v"], causal=causal)
    _check_against_oracle(_f64(o), _f64(lse), O, LSE, what)
    refs = oa.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], causal=causal)
    for name, got, ref in zip(("dQ", "dK", "dV"), (dq, dk, dv), refs):
        mag = np.max(np.abs(ref))
        err = np.max(np.abs(_f64(got) - ref))
        assert err <= G_TOL * mag, f"{what} {name} {err:.3e} > {G_TOL * mag:.3e}"


def test_split_chosen_automatically_for_narrow_launches():
    """fa.fwd picks fa_fwd_split_count's split for a launch that cannot fill
    the device (one query row per head against 16K keys) and gives the
    unsplit result; sampled rows of every head also match the oracle."""
    _say("case split auto decode")
    from io_aware_exact_02_amd import _lib
    assert _lib.load().fa_fwd_split_count(1, 16, 1, 16384, 64, 1) > 1
    inp = _inputs(1, 1, 16384, 16, 64, "bf16", 9400)
    dev = torch.device("cuda")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, causal=True)
    o1, lse1 = fa.fwd(q, k, v, causal=True, num_splits=1)
    torch.cuda.synchronize()
    vmax = float(np.max(np.abs(_f64(inp["v"]))))
    _check_against_unsplit(_f64(o), _f64(lse), _f64(o1), _f64(lse1), vmax, "bf16", "auto decode")
    for h in range(16):
        r = oa.attention_rows(inp["q"], inp["k"], inp["v"], inp["do"], 0, h, [0], causal=True)
        assert np.max(np.abs(_f64(o)[0, [0], h] - r["O"])) <= O_TOL, f"h{h} O"
        assert np.max(np.abs(_f64(lse)[0, h, [0]] - r["LSE"])) <= LSE_TOL, f"h{h} LSE"


def test_split_long_context_sampled_rows():
    """A chunk of 512 queries at the end of a 16K-key causal context, 8
    heads, 8 splits, against the row-sampled oracle."""
    _say("case split chunk 512 of 16K")
    Nq, Nk, H = 512, 16384, 8
    inp = _inputs(1, Nq, Nk, H, 64, "bf16", 9500)
    dev = torch.device("cuda")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, causal=True, num_splits=8)
    torch.cuda.synchronize()
    o, lse = _f64(o), _f64(lse)
    rows = sample_rows(Nq, 48, seed=9501)
    for h in range(H):
        r = oa.attention_rows(inp["q"], inp["k"], inp["v"], inp["do"], 0, h, rows, causal=True)
        assert np.max(np.abs(o[0, rows, h] - r["O"])) <= O_TOL, f"h{h} O"
        assert np.max(np.abs(lse[0, h, rows] - r["LSE"])) <= LSE_TOL, f"h{h} LSE"


def test_split_packed_inputs_and_strided_output():
    """Packed qkv views (n-stride 3*H*D) in, a strided view of a wider tensor
    out: the merge kernel writes through the caller's output strides."""
    _say("case split packed/strided")
    B, N, H, D = 2, 700, 3, 64
    inp = random_qkv(B, N, H, D, "bf16", 9600, layout="packed")
    dev = torch.device("cuda")
    qkv = inp["qkv"].to(dev)
    q, k, v = qkv.unbind(dim=2)
    wide = torch.full((B, N, H, 2 * D), float("nan"), dtype=torch.bfloat16, device=dev)
    out = wide[..., D:]
    o, lse = fa.fwd(q, k, v, causal=True, num_splits=3, out=out)
    o1, lse1 = fa.fwd(q, k, v, causal=True, num_splits=1)
    torch.cuda.synchronize()
    assert o.data_ptr() == out.data_ptr()
    assert torch.isnan(wide[..., :D]).all(), "wrote outside the output view"
    qc, kc, vc = (inp["qkv"][:, :, i] for i in range(3))
    O, LSE = oa.attention_forward(qc, kc, vc, causal=True)
    _check_against_oracle(_f64(o), _f64(lse), O, LSE, "packed split")
    vmax = float(np.max(np.abs(_f64(vc))))
    _check_against_unsplit(_f64(o), _f64(lse), _f64(o1), _f64(lse1), vmax, "bf16", "packed split")


def test_split_graph_replay_matches_eager():
    """The key-split forward (partials in a workspace allocated at capture,
    then the merge) captured in a HIP graph: every replay, with stale outputs
    and eager work in between, equals the eager result bit for bit."""
    _say("case split graph replay")
    inp = _inputs(1, 64, 4096, 4, 64, "bf16", 9700)
    dev = torch.device("cuda")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o_e, lse_e = fa.fwd(q, k, v, causal=True, num_splits=4)
    torch.cuda.synchronize()
    o, lse = torch.empty_like(o_e), torch.empty_like(lse_e)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fa.fwd(q, k, v, causal=True, num_splits=4, out=o, lse=lse)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fwd(q, k, v, causal=True, num_splits=4, out=o, lse=lse)
    for rep in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_e) and torch.equal(lse, lse_e), f"replay {rep}"
        _ = torch.cos(q.float()).sum()
        torch.cuda.synchronize()

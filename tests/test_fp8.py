"""GPU parity of the FP8 forward (fa_fwd_fp8 through the binding) against the
FP8 oracle, on the same E4M3 codes and descale factors.

Two bars, both derived from the arithmetic (the pages state no FP8 recipe):

* Exact-weight inputs: every softmax weight is a power of two in
  [2^-8, 2^8], which E4M3 holds exactly, so rounding P changes nothing and
  the kernel must match exact attention up to fp32 accumulation and the
  output rounding: |O - O_ref| <= 2^-8 |O_ref| + 1e-4 max|v|.  Any slip in
  the operand layouts (a key paired with the wrong V row, a wrong byte
  order) fails this bar.
* Random N(0,1) inputs quantized per (batch, head): |O - O_ref| within the
  oracle's elementwise bound for rounding P to E4M3.

LSE max-abs <= 1e-3 in both (the LSE comes from the unrounded fp32
weights).  Rows that see no key must be exactly O = 0, LSE = -inf.
"""

import sys

import numpy as np
import pytest
import torch

import io_aware_exact_02_amd as fa
from oracle import fp8 as o8
from workloads import fp8_exact_weight_inputs, fp8_random_inputs, sample_rows

pytestmark = pytest.mark.gpu

LSE_TOL = 1e-3
OUT = {"bf16": torch.bfloat16, "f16": torch.float16}


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _run(d, causal, scale=None, out="bf16"):
    dev = torch.device("cuda")
    q, k, v = (d[n].to(dev) for n in ("q", "k", "v"))
    ds = [d["descale_" + n].to(dev) for n in ("q", "k", "v")]
    o, lse = fa.fwd_fp8(q, k, v, *ds, causal=causal, softmax_scale=scale,
                        out_dtype=OUT[out])
    torch.cuda.synchronize()
    return _f64(o), _f64(lse)


def _args(d):
    return d["q"], d["k"], d["v"], d["descale_q"], d["descale_k"], d["descale_v"]


def _check_lse_and_empty(o, lse, O, LSE, what):
    empty = np.isneginf(LSE)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: empty rows differ"
    if empty.any():
        assert np.all(o[np.transpose(empty, (0, 2, 1))] == 0.0), f"{what}: empty rows not 0"
    assert np.all(np.isfinite(o)), what
    if (~empty).any():
        el = np.max(np.abs(lse[~empty] - LSE[~empty]))
        assert el <= LSE_TOL, f"{what}: LSE max-abs {el:.3e}"


LENGTHS = [(1, 1), (17, 17), (64, 64), (128, 128), (129, 129), (300, 300), (513, 513),
           (64, 300), (300, 64), (1, 200)]


@pytest.mark.parametrize("out", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Nq,Nk", LENGTHS)
def test_exact_weights(Nq, Nk, D, causal, out):
    what = f"fp8 exact Nq={Nq} Nk={Nk} D={D} causal={causal} {out}"
    _say("case", what)
    d = fp8_exact_weight_inputs(2, Nq, Nk, 3, D, 8000 + Nq + 7 * Nk + D)
    o, lse = _run(d, causal, d["scale"], out)
    O, LSE = o8.attention_forward_fp8(*_args(d), causal=causal, scale=d["scale"])
    _check_lse_and_empty(o, lse, O, LSE, what)
    vmax = np.abs(o8._descaled(d["v"], d["descale_v"])).max()
    err = np.abs(o - O) - (2.0 ** -8 * np.abs(O) + 1e-4 * vmax)
    assert np.all(err <= 0), f"{what}: O over the bar by {np.max(err):.3e}"


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Nq,Nk", LENGTHS)
def test_random_within_bound(Nq, Nk, D, causal):
    what = f"fp8 random Nq={Nq} Nk={Nk} D={D} causal={causal}"
    _say("case", what)
    d = fp8_random_inputs(2, Nq, Nk, 3, D, 8100 + Nq + 7 * Nk + D)
    o, lse = _run(d, causal)
    O, LSE = o8.attention_forward_fp8(*_args(d), causal=causal)
    _check_lse_and_empty(o, lse, O, LSE, what)
    E = o8.fp8_output_bound(*_args(d), causal=causal)
    over = np.abs(o - O) - E
    assert np.all(over <= 0), f"{what}: O over the bound by {np.max(over):.3e}"


@pytest.mark.parametrize("scale", [0.0, -0.3, 0.5])
def test_scale_and_descale_signs(scale):
    """A negative scale, and a negative descale factor on one head, flip the
    scores; a zero scale gives uniform weights."""
    _say("case fp8 scale", scale)
    d = fp8_random_inputs(1, 150, 150, 2, 64, 8200)
    d["descale_k"] = d["descale_k"].clone()
    d["descale_k"][0, 1] *= -1.0
    o, lse = _run(d, False, scale)
    O, LSE = o8.attention_forward_fp8(*_args(d), scale=scale)
    _check_lse_and_empty(o, lse, O, LSE, f"scale {scale}")
    E = o8.fp8_output_bound(*_args(d), scale=scale)
    assert np.all(np.abs(o - O) <= E)


def test_no_descale_means_one():
    _say("case fp8 descale None")
    d = fp8_random_inputs(1, 100, 100, 2, 128, 8300, per_head_scale=False)
    dev = torch.device("cuda")
    q, k, v = (d[n].to(dev) for n in ("q", "k", "v"))
    o, lse = fa.fwd_fp8(q, k, v)
    ones = torch.ones((1, 2))
    O, LSE = o8.attention_forward_fp8(d["q"], d["k"], d["v"], ones, ones, ones)
    torch.cuda.synchronize()
    _check_lse_and_empty(_f64(o), _f64(lse), O, LSE, "no descale")
    E = o8.fp8_output_bound(d["q"], d["k"], d["v"], ones, ones, ones)
    assert np.all(np.abs(_f64(o) - O) <= E)


def test_float8_dtype_and_strided_inputs():
    """torch.float8_e4m3fn tensors and strided [B, H, N, D] views give the
    same result as contiguous uint8 codes."""
    _say("case fp8 dtypes and strides")
    d = fp8_random_inputs(2, 200, 200, 4, 64, 8400)
    dev = torch.device("cuda")
    ds = [d["descale_" + n].to(dev) for n in ("q", "k", "v")]
    base = fa.fwd_fp8(*(d[n].to(dev) for n in ("q", "k", "v")), *ds, causal=True)
    f8 = [d[n].to(dev).view(torch.float8_e4m3fn) for n in ("q", "k", "v")]
    alt = fa.fwd_fp8(*f8, *ds, causal=True)
    bhnd = [d[n].to(dev).transpose(1, 2).contiguous().transpose(1, 2) for n in ("q", "k", "v")]
    alt2 = fa.fwd_fp8(*bhnd, *ds, causal=True)
    torch.cuda.synchronize()
    for a in (alt, alt2):
        assert torch.equal(a[0], base[0]) and torch.equal(a[1], base[1])


def test_determinism():
    _say("case fp8 determinism")
    d = fp8_random_inputs(1, 1000, 1000, 4, 128, 8500)
    r1 = _run(d, True)
    r2 = _run(d, True)
    assert np.array_equal(r1[0], r2[0]) and np.array_equal(r1[1], r2[1])


@pytest.mark.parametrize("name,B,H,N,D", [("c4 shape", 1, 8, 8192, 128),
                                          ("c5 shape", 1, 16, 16384, 64)])
def test_full_size_sampled(name, B, H, N, D):
    """The long causal shapes of the 16-bit workloads with FP8 inputs: O and
    LSE at 128 sampled rows of every head against the row-sampled oracle."""
    _say("case fp8", name)
    d = fp8_random_inputs(B, N, N, H, D, 8600 + N)
    o, lse = _run(d, True)
    rows = sample_rows(N, 128, seed=8700 + N)
    for h in range(H):
        r = o8.fp8_rows(*_args(d), 0, h, rows, causal=True)
        assert np.max(np.abs(lse[0, h, rows] - r["LSE"])) <= LSE_TOL, f"{name} h{h} LSE"
        assert np.all(np.abs(o[0, rows, h] - r["O"]) <= r["bound"]), f"{name} h{h} O"


@pytest.mark.parametrize("D,causal", [(64, True), (128, True), (128, False)])
def test_twelve_heads(D, causal):
    """B*H = 12, not a multiple of the 8 XCDs: the workgroup id -> (head,
    block) mapping with ids past the last block.  Exact-weight inputs,
    several blocks and a ragged tail."""
    what = f"fp8 B=2 H=6 D={D} causal={causal}"
    _say("case", what)
    d = fp8_exact_weight_inputs(2, 1100, 1100, 6, D, 8700 + D + int(causal))
    o, lse = _run(d, causal, d["scale"])
    O, LSE = o8.attention_forward_fp8(*_args(d), causal=causal, scale=d["scale"])
    _check_lse_and_empty(o, lse, O, LSE, what)
    vmax = np.abs(o8._descaled(d["v"], d["descale_v"])).max()
    assert np.all(np.abs(o - O) <= 2.0 ** -8 * np.abs(O) + 1e-4 * vmax), what


@pytest.mark.parametrize("Nq,Nk", [(1024, 1024), (1100, 1100), (1100, 1500), (1500, 1100)])
def test_split_paired_head_dim_128(Nq, Nk):
    """Causal head_dim-128 launches whose workgroups all fit on the device at
    once run the split, paired form (two key groups merged in LDS, query
    blocks i and n-1-i in one workgroup): even and odd block counts, and
    rows that see no key.  Exact-weight inputs (tight bar) and random
    inputs (the oracle's bound)."""
    what = f"fp8 split Nq={Nq} Nk={Nk}"
    _say("case", what)
    d = fp8_exact_weight_inputs(1, Nq, Nk, 2, 128, 8800 + Nq + Nk)
    o, lse = _run(d, True, d["scale"])
    O, LSE = o8.attention_forward_fp8(*_args(d), causal=True, scale=d["scale"])
    _check_lse_and_empty(o, lse, O, LSE, what)
    vmax = np.abs(o8._descaled(d["v"], d["descale_v"])).max()
    assert np.all(np.abs(o - O) <= 2.0 ** -8 * np.abs(O) + 1e-4 * vmax), what
    d = fp8_random_inputs(1, Nq, Nk, 2, 128, 8900 + Nq + Nk)
    o, lse = _run(d, True)
    O, LSE = o8.attention_forward_fp8(*_args(d), causal=True)
    _check_lse_and_empty(o, lse, O, LSE, what)
    assert np.all(np.abs(o - O) <= o8.fp8_output_bound(*_args(d), causal=True)), what


def _fp8_random_cases(count, seed):
    import random
    rnd = random.Random(seed)
    lengths = [1, 2, 31, 64, 65, 127, 128, 129, 200, 333, 513]
    return [(i, rnd.randint(1, 3), rnd.randint(1, 4), rnd.choice(lengths), rnd.choice(lengths),
             rnd.choice([64, 128]), rnd.random() < 0.5, rnd.choice(["bf16", "f16"]),
             rnd.choice([None, 0.05, -0.09])) for i in range(count)]


FP8_RANDOM = _fp8_random_cases(24, seed=20261204)


@pytest.mark.parametrize("i,B,H,Nq,Nk,D,causal,out,scale", FP8_RANDOM,
                         ids=[f"case{c[0]}" for c in FP8_RANDOM])
def test_random_sample(i, B, H, Nq, Nk, D, causal, out, scale):
    """A seeded random sample crossing lengths, head_dim, mask, output type
    and scale (including negative ones) with per-head quantized inputs: O
    within the oracle's elementwise bound, LSE <= 1e-3, empty rows exact."""
    what = f"fp8 random {i}: B={B} H={H} Nq={Nq} Nk={Nk} D={D} causal={causal} {out} scale={scale}"
    _say("case", what)
    d = fp8_random_inputs(B, Nq, Nk, H, D, 12000 + i)
    o, lse = _run(d, causal, scale, out)
    O, LSE = o8.attention_forward_fp8(*_args(d), causal=causal, scale=scale)
    _check_lse_and_empty(o, lse, O, LSE, what)
    E = o8.fp8_output_bound(*_args(d), causal=causal, scale=scale)
    over = np.abs(o - O) - E
    assert np.all(over <= 0), f"{what}: O over the bound by {np.max(over):.3e}"

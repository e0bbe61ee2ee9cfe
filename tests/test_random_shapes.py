"""GPU parity on a seeded random sample of problem shapes and options.

Each case draws B, H, N_q, N_k, head_dim, mask, input type, scale and key
split count from a fixed generator, runs the forward (fa.fwd, key-split
when drawn) and the backward through the binding, and compares O, LSE,
dQ, dK and dV with the fp64 oracle: LSE max-abs <= 1e-3 (rows that see no
key exactly O = 0, LSE = -inf), each gradient max-abs <= 5e-2 *
max|reference|, and O element by element within 1e-2 where |O| < 2 and,
where |O| >= 2, within 1e-2 plus 2^-8 |O| for bf16 (2^-11 |O| for fp16):
the rounding of the exact value to the output type (half a spacing, 2^-9
|O|) plus that of the softmax weights before the P V product (at most
2^-9 max|v|).  Below |O| = 2 the output's rounding costs at most 3.9e-3 and
the plain bar keeps its margin; at |O| >= 4 no bf16 value need lie within
1e-2 of the exact one (the first run of this sample failed the plain bar
exactly at elements the kernel rounded to bf16(O) itself), and in [2, 4)
the two roundings together reach 1.0e-2 (seen once in this sample).  Cases
with |O| >= 2 report their error per |O| band.  The sample crosses options
that the grid tests take one at a time (unequal lengths with a negative
scale and a key split, ragged tails on both sides, one-row problems).
"""

import random
import sys

import numpy as np
import pytest
import torch

import io_aware_exact_02_amd as fa
import oband
from oracle import attention as oa
from workloads import random_qkv

pytestmark = pytest.mark.gpu

O_TOL = 1e-2
RND = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
LSE_TOL = 1e-3
G_TOL = 5e-2


def _draw_cases(count, seed):
    rnd = random.Random(seed)
    lengths = [1, 2, 31, 64, 65, 127, 200, 256, 333, 513, 700]
    cases = []
    for i in range(count):
        nq, nk = rnd.choice(lengths), rnd.choice(lengths)
        splits = rnd.choice([1, 1, 2, 3, 5]) if nk > 128 else 1
        cases.append((i, rnd.randint(1, 3), rnd.randint(1, 4), nq, nk, rnd.choice([64, 128]),
                      rnd.random() < 0.5, rnd.choice(["bf16", "f16"]),
                      rnd.choice([None, None, 0.3, -0.7]), splits))
    return cases


CASES = _draw_cases(48, seed=20261203)


@pytest.mark.parametrize("i,B,H,Nq,Nk,D,causal,dtype,scale,splits", CASES,
                         ids=[f"case{c[0]}" for c in CASES])
def test_random_shape(i, B, H, Nq, Nk, D, causal, dtype, scale, splits):
    what = (f"random case {i}: B={B} H={H} Nq={Nq} Nk={Nk} D={D} causal={causal} {dtype} "
            f"scale={scale} splits={splits}")
    print("case", what, flush=True)
    sys.stdout.flush()
    a = random_qkv(B, Nq, H, D, dtype, 11000 + 2 * i)
    b = random_qkv(B, Nk, H, D, dtype, 11001 + 2 * i)
    dev = torch.device("cuda")
    q, do = a["q"].to(dev), a["do"].to(dev)
    k, v = b["k"].to(dev), b["v"].to(dev)
    o, lse = fa.fwd(q, k, v, causal=causal, softmax_scale=scale, num_splits=splits)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal, softmax_scale=scale)
    torch.cuda.synchronize()
    f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()
    o, lse = f64(o), f64(lse)
    O, LSE = oa.attention_forward(a["q"], b["k"], b["v"], causal=causal, scale=scale)
    empty = np.isneginf(LSE)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: empty rows differ"
    if empty.any():
        assert np.all(o[np.transpose(empty, (0, 2, 1))] == 0.0), f"{what}: empty rows not 0"
    assert np.all(np.isfinite(o)), what
    err = np.abs(o - O)
    small = np.abs(O) < 2.0
    if not small.all():
        oband.record(f"random case {i}", o, O)
    if small.any():
        es = np.max(err[small])
        assert es <= O_TOL, f"{what}: O max-abs {es:.3e} where |O| < 2"
    over = err - (O_TOL + RND[dtype] * np.abs(O))
    assert np.all(over <= 0), f"{what}: O over the bar by {np.max(over):.3e}"
    if (~empty).any():
        el = np.max(np.abs(lse[~empty] - LSE[~empty]))
        assert el <= LSE_TOL, f"{what}: LSE {el:.3e}"
    refs = oa.attention_backward(a["q"], b["k"], b["v"], a["do"], causal=causal, scale=scale)
    for name, got, ref in zip(("dQ", "dK", "dV"), (dq, dk, dv), refs):
        got = f64(got)
        assert np.all(np.isfinite(got)), f"{what}: {name} not finite"
        mag = np.max(np.abs(ref))
        bound = G_TOL * mag if mag > 0 else 1e-3
        err = np.max(np.abs(got - ref))
        assert err <= bound, f"{what}: {name} {err:.3e} > {bound:.3e}"

"""GPU race detection for the kernels' LDS use.

Two checks:

* LDS poisoning: ``libfa_poison.so`` is the same library built with
  FA_POISON_LDS=1, whose kernels fill every LDS array with NaN bits when a
  workgroup starts.  A kernel that reads LDS it has not written (a missing
  barrier, a tile that is not loaded, a buffer reused too early) then
  returns NaN instead of stale data.  The cases below run every launch form
  -- 4- and 8-wave head_dim-64 forwards, the head_dim-128 plain and split
  forms, key splits, the vector-unit forward of one or two rows, the FP8
  forward, the backward with and without query
  segments, ragged tails and head counts off the XCD grid -- through the
  poisoned build and check them against the oracle.
* Determinism: three runs of each tile configuration give bitwise equal O,
  LSE, dQ, dK and dV (a race on LDS shows up as drift between runs).
"""

import sys

import numpy as np
import pytest
import torch

import io_aware_exact_02_amd as fa
from io_aware_exact_02_amd import _lib
from oracle import attention as oa
from oracle import fp8 as o8
from workloads import fp8_exact_weight_inputs, random_qkv, sample_rows

pytestmark = pytest.mark.gpu

O_TOL, LSE_TOL, G_TOL = 1e-2, 1e-3, 5e-2


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture
def poisoned(monkeypatch):
    """Route the binding through libfa_poison.so for one test."""
    lib = _lib.open_library(_lib.POISON_LIB_PATH)
    monkeypatch.setattr(_lib, "_lib", lib)
    return lib


def _f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _run(inp, causal, splits=None):
    dev = torch.device("cuda")
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=causal, num_splits=splits)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal)
    torch.cuda.synchronize()
    return {"O": _f64(o), "LSE": _f64(lse), "dQ": _f64(dq), "dK": _f64(dk), "dV": _f64(dv)}


def _grad_ok(name, got, ref, what):
    assert np.all(np.isfinite(got)), f"{what}: {name} not finite"
    mag = np.max(np.abs(ref))
    bound = G_TOL * mag if mag > 0 else 1e-3
    err = np.max(np.abs(got - ref))
    assert err <= bound, f"{what}: {name} {err:.3e} > {bound:.3e}"


def _check_full(inp, causal, what, splits=None):
    got = _run(inp, causal, splits)
    O, LSE = oa.attention_forward(inp["q"], inp["k"], inp["v"], causal=causal)
    assert np.all(np.isfinite(got["O"])) and np.all(np.isfinite(got["LSE"])), what
    assert np.max(np.abs(got["O"] - O)) <= O_TOL, f"{what}: O"
    assert np.max(np.abs(got["LSE"] - LSE)) <= LSE_TOL, f"{what}: LSE"
    refs = oa.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], causal=causal)
    for name, ref in zip(("dQ", "dK", "dV"), refs):
        _grad_ok(name, got[name], ref, what)


def _check_rows(inp, causal, what, nrows=48):
    """Large launches: O, LSE, dQ at sampled rows of every head; dK, dV in
    full on the first head."""
    got = _run(inp, causal)
    B, N, H, _ = inp["q"].shape
    for name in ("O", "LSE", "dQ", "dK", "dV"):
        assert np.all(np.isfinite(got[name])), f"{what}: {name} not finite"
    rows = sample_rows(N, nrows, seed=N + H)
    for b in range(B):
        for h in range(H):
            r = oa.attention_rows(inp["q"], inp["k"], inp["v"], inp["do"], b, h, rows,
                                  causal=causal)
            assert np.max(np.abs(got["O"][b, rows, h] - r["O"])) <= O_TOL, f"{what}: O b{b} h{h}"
            assert np.max(np.abs(got["LSE"][b, h, rows] - r["LSE"])) <= LSE_TOL, f"{what}: LSE"
            _grad_ok("dQ", got["dQ"][b, rows, h], r["dQ"], f"{what} b{b} h{h}")
    _, dK, dV = oa.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], causal=causal,
                                      heads=[(0, 0)])
    _grad_ok("dK", got["dK"][0, :, 0], dK[0, :, 0], what)
    _grad_ok("dV", got["dV"][0, :, 0], dV[0, :, 0], what)


# ------------------------------------------------------------ LDS poisoning

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("N", [1, 17, 129, 300])
def test_poisoned_small(poisoned, N, D, causal):
    """4-wave forwards, the head_dim-128 split form (non-causal), the
    backward with query segments (causal, and non-causal past one query
    tile) and without, ragged tails."""
    what = f"poisoned N={N} D={D} causal={causal}"
    _say("case", what)
    _check_full(random_qkv(2, N, 3, D, "bf16", seed=9100 + N + D), causal, what)


@pytest.mark.parametrize("Nq,Nk,D,causal,splits", [(1, 3000, 64, True, 5), (2, 1500, 128, False, 3),
                                                 (2, 2, 64, True, 1)])
def test_poisoned_decode(poisoned, Nq, Nk, D, causal, splits):
    """The vector-unit forward of one or two rows (its LDS combine of the
    four waves), split and unsplit, and the backward after it."""
    what = f"poisoned decode Nq={Nq} Nk={Nk} D={D} causal={causal} splits={splits}"
    _say("case", what)
    a = random_qkv(1, Nq, 3, D, "bf16", seed=9250 + Nk + D)
    b = random_qkv(1, Nk, 3, D, "bf16", seed=9251 + Nk + D)
    inp = {"q": a["q"], "do": a["do"], "k": b["k"], "v": b["v"]}
    got = _run(inp, causal, splits)
    O, LSE = oa.attention_forward(inp["q"], inp["k"], inp["v"], causal=causal)
    assert np.max(np.abs(got["O"] - O)) <= O_TOL, f"{what}: O"
    assert np.max(np.abs(got["LSE"] - LSE)) <= LSE_TOL, f"{what}: LSE"
    refs = oa.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], causal=causal)
    for name, ref in zip(("dQ", "dK", "dV"), refs):
        _grad_ok(name, got[name], ref, what)


@pytest.mark.parametrize("D,causal,splits", [(64, True, 3), (128, False, 2), (64, False, 5)])
def test_poisoned_key_splits(poisoned, D, causal, splits):
    what = f"poisoned key splits D={D} causal={causal} splits={splits}"
    _say("case", what)
    _check_full(random_qkv(1, 700, 3, D, "f16", seed=9200 + D + splits), causal, what, splits)


def test_poisoned_eight_wave_forward(poisoned):
    """B*H*ceil(N/256) = 1024: the causal 8-wave head_dim-64 forward
    (interleaved pipeline steps) and the unsegmented backward."""
    what = "poisoned B=8 H=16 N=2048 D=64 causal"
    _say("case", what)
    _check_rows(random_qkv(8, 2048, 16, 64, "bf16", seed=9300), True, what, nrows=16)


def test_poisoned_eight_wave_forward_non_causal(poisoned):
    """B*H*ceil(N/256) = 512, non-causal: the 8-wave head_dim-64 forward."""
    what = "poisoned B=4 H=16 N=2048 D=64 non-causal"
    _say("case", what)
    _check_rows(random_qkv(4, 2048, 16, 64, "bf16", seed=9310), False, what, nrows=16)


@pytest.mark.parametrize("N", [1100, 1500])
def test_poisoned_paired_head_dim_128(poisoned, N):
    """Causal head_dim 128 with few workgroups: the split, paired forward
    (LDS merge of two key groups) with an odd and an even block count."""
    what = f"poisoned paired D=128 N={N}"
    _say("case", what)
    _check_full(random_qkv(1, N, 2, 128, "bf16", seed=9400 + N), True, what)


def test_poisoned_head_dim_128_eight_waves(poisoned):
    """B*H*ceil(N/256) = 512 at head_dim 128, causal: the plain 8-wave
    forward."""
    what = "poisoned B=2 H=16 N=4096 D=128 causal"
    _say("case", what)
    _check_rows(random_qkv(2, 4096, 16, 128, "bf16", seed=9450), True, what, nrows=8)


def test_poisoned_heads_off_xcd_grid(poisoned):
    what = "poisoned B=1 H=3 N=520 D=64 causal"
    _say("case", what)
    _check_full(random_qkv(1, 520, 3, 64, "bf16", seed=9500), True, what)


@pytest.mark.parametrize("D,causal,N", [(64, True, 300), (128, True, 1100), (128, False, 300)])
def test_poisoned_fp8(poisoned, D, causal, N):
    """The FP8 forward (4-wave, and the split paired form at head_dim 128)."""
    what = f"poisoned fp8 D={D} causal={causal} N={N}"
    _say("case", what)
    d = fp8_exact_weight_inputs(1, N, N, 2, D, 9600 + D + N)
    dev = torch.device("cuda")
    q, k, v = (d[n].to(dev) for n in ("q", "k", "v"))
    ds = [d["descale_" + n].to(dev) for n in ("q", "k", "v")]
    o, lse = fa.fwd_fp8(q, k, v, *ds, causal=causal, softmax_scale=d["scale"])
    torch.cuda.synchronize()
    o, lse = _f64(o), _f64(lse)
    args = (d["q"], d["k"], d["v"], d["descale_q"], d["descale_k"], d["descale_v"])
    O, LSE = o8.attention_forward_fp8(*args, causal=causal, scale=d["scale"])
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), what
    vmax = np.abs(o8._descaled(d["v"], d["descale_v"])).max()
    assert np.all(np.abs(o - O) <= 2.0 ** -8 * np.abs(O) + 1e-4 * vmax), what
    assert np.max(np.abs(lse - LSE)) <= LSE_TOL, what


# ------------------------------------------------------------ determinism

TILE_CONFIGS = [
    # (label, B, H, N, D, causal): the launch form each one selects
    ("d64 4-wave fwd, unsegmented bwd", 4, 12, 1024, 64, False),
    ("d64 segmented non-causal bwd", 2, 4, 1000, 64, False),
    ("d64 8-wave fwd", 8, 16, 2048, 64, True),
    ("d64 segmented bwd", 1, 2, 3000, 64, True),
    ("d128 paired fwd, segmented bwd", 1, 4, 2048, 128, True),
    ("d128 4-wave fwd", 2, 4, 900, 128, True),
    ("d128 split non-causal fwd", 2, 4, 1000, 128, False),
]


@pytest.mark.parametrize("label,B,H,N,D,causal", TILE_CONFIGS, ids=[c[0] for c in TILE_CONFIGS])
def test_three_runs_bitwise(label, B, H, N, D, causal):
    _say("case determinism", label)
    inp = random_qkv(B, N, H, D, "bf16", seed=9700 + N + D)
    runs = [_run(inp, causal) for _ in range(3)]
    for key in ("O", "LSE", "dQ", "dK", "dV"):
        for r in runs[1:]:
            assert np.array_equal(runs[0][key], r[key], equal_nan=True), f"{label}: {key}"

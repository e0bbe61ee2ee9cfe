"""The HIP path under HIP graph capture and at the long end of N.

* Graph: fwd and bwd of a head_dim-64 causal problem and an FP8 forward are
  captured once and replayed several times, with eager work and
  synchronisations between replays; every replay must equal the eager
  result bit for bit (the kernels clear their own workspace; nothing in the
  path records a memset).
* Long N: B=1 H=1 N=65536 D=64 causal; O, LSE and dQ at rows sampled over
  the whole range (first, middle and last tiles included) against the
  row-sampled oracle; dK and dV must be finite.
"""

import sys

import numpy as np
import pytest
import torch

import io_aware_exact_02_amd as fa
from oracle import attention as oa
from workloads import fp8_random_inputs, random_qkv, sample_rows

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_graph_replay_matches_eager():
    _say("case graph replay")
    dev = torch.device("cuda")
    inp = random_qkv(1, 1000, 4, 64, "bf16", seed=9300)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o_e, lse_e = fa.fwd(q, k, v, causal=True)
    dq_e, dk_e, dv_e = fa.bwd(q, k, v, o_e, lse_e, do, causal=True)
    d8 = fp8_random_inputs(1, 600, 600, 2, 128, 9301)
    q8, k8, v8 = (d8[n].to(dev) for n in ("q", "k", "v"))
    ds8 = [d8["descale_" + n].to(dev) for n in ("q", "k", "v")]
    o8_e, lse8_e = fa.fwd_fp8(q8, k8, v8, *ds8, causal=True)
    torch.cuda.synchronize()

    ws = torch.empty(fa.workspace_bytes(1, 4, 1000, 64), dtype=torch.uint8, device=dev)
    o = torch.empty_like(o_e)
    lse = torch.empty_like(lse_e)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    o8 = torch.empty_like(o8_e)
    lse8 = torch.empty_like(lse8_e)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up on the capture stream
        fa.fwd(q, k, v, causal=True, out=o, lse=lse)
        fa.bwd(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws)
        fa.fwd_fp8(q8, k8, v8, *ds8, causal=True, out=o8, lse=lse8)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fwd(q, k, v, causal=True, out=o, lse=lse)
        fa.bwd(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws)
        fa.fwd_fp8(q8, k8, v8, *ds8, causal=True, out=o8, lse=lse8)
    for rep in range(4):
        for t in (o, lse, dq, dk, dv, o8, lse8):
            t.fill_(float("nan") if t.is_floating_point() else 0)
        ws.fill_(0xAB)                     # stale workspace contents
        g.replay()
        torch.cuda.synchronize()
        for got, ref in ((o, o_e), (lse, lse_e), (dq, dq_e), (dk, dk_e), (dv, dv_e),
                         (o8, o8_e), (lse8, lse8_e)):
            assert torch.equal(got, ref), f"replay {rep}"
        _ = torch.sin(q.float()).sum()   # eager work between replays
        torch.cuda.synchronize()


def test_long_sequence_sampled():
    """N = 65536 (one head): far beyond the other cases; rows sampled over the
    whole range, including the last tile."""
    N = 65536
    _say("case long N", N)
    dev = torch.device("cuda")
    inp = random_qkv(1, N, 1, 64, "bf16", seed=9400)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=True)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    rows = sample_rows(N, 64, seed=9401)
    r = oa.attention_rows(inp["q"], inp["k"], inp["v"], inp["do"], 0, 0, rows, causal=True)
    got_o = o[0, rows, 0].double().cpu().numpy()
    assert np.max(np.abs(got_o - r["O"])) <= 1e-2
    assert np.max(np.abs(lse[0, 0, rows].double().cpu().numpy() - r["LSE"])) <= 1e-3
    got_dq = dq[0, rows, 0].double().cpu().numpy()
    assert np.max(np.abs(got_dq - r["dQ"])) <= 5e-2 * np.max(np.abs(r["dQ"]))
    assert torch.isfinite(dk).all() and torch.isfinite(dv).all()

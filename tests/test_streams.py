"""Concurrent calls on different streams.

The library keeps no state between calls (every buffer, workspace included,
belongs to the caller), so independent problems enqueued on separate
streams at once must give exactly what they give one after the other.
Every path used here is bitwise repeatable (integer dQ accumulation, fixed
merge orders), so the comparison is bit for bit.  fa_bwd_noalloc is left
out: its calls share one scratch array per device by design.
"""

import sys

import pytest
import torch

import io_aware_exact_02_amd as fa
from workloads import random_qkv

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _problems(dev):
    a = random_qkv(2, 1500, 4, 64, "bf16", seed=9810)
    b = random_qkv(1, 1200, 3, 128, "f16", seed=9811)
    c = random_qkv(2, 2, 4, 128, "bf16", seed=9812)
    ck = random_qkv(2, 3000, 4, 128, "bf16", seed=9813)
    return [
        ("fwd+bwd d64 causal", {n: a[n].to(dev) for n in ("q", "k", "v", "do")}, True, None),
        ("fwd+bwd d128 key splits", {n: b[n].to(dev) for n in ("q", "k", "v", "do")}, False, 3),
        ("decode d128", {"q": c["q"].to(dev), "do": c["do"].to(dev), "k": ck["k"].to(dev),
                         "v": ck["v"].to(dev)}, True, None),
    ]


def _run(p, causal, splits):
    o, lse = fa.fwd(p["q"], p["k"], p["v"], causal=causal, num_splits=splits)
    dq, dk, dv = fa.bwd(p["q"], p["k"], p["v"], o, lse, p["do"], causal=causal)
    return o, lse, dq, dk, dv


def test_concurrent_streams_match_sequential():
    _say("case concurrent streams")
    dev = torch.device("cuda")
    probs = _problems(dev)
    ref = [_run(p, c, s) for _, p, c, s in probs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in probs]
    for rep in range(3):
        outs = [None] * len(probs)
        for i, ((_, p, c, s), st) in enumerate(zip(probs, streams)):
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                outs[i] = _run(p, c, s)
        for st in streams:
            torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        for (name, _, _, _), got, want in zip(probs, outs, ref):
            for label, g, w in zip(("O", "LSE", "dQ", "dK", "dV"), got, want):
                assert torch.equal(g, w), f"rep {rep} {name}: {label} differs from sequential"

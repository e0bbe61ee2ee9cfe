#!/usr/bin/env python3
"""Benchmark of the fused attention hot path on one MI355X.

Metric: attention forward + backward throughput in TFLOP/s (and as a
fraction of the dense bf16/fp16 MFMA peak) over the sequence-length sweep
N = 512 .. 16384.  One step runs fa_fwd and the three backward kernels once
for each of the four workloads

    c2  B=2  H=12 N=512   D=64  fp16 packed qkv, non-causal
    c3  B=2  H=12 N=2048  D=64  fp16 packed qkv, non-causal
    c4  B=1  H=8  N=8192  D=128 bf16 [B,N,H,D],  causal
    c5  B=1  H=16 N=16384 D=64  bf16 [B,N,H,D],  causal

with seeded N(0,1) inputs already resident in HBM.  FLOPs follow the usual
convention: forward 4*B*H*N^2*D, backward 2.5x that (five products against
two), both halved for causal masking.

Prints ONE JSON line.  Besides the headline value it carries
  roofline     : the dominant kernel (the dK/dV backward kernel at c5) timed
                 with HIP events on its own stream inside the timed region,
                 against the 2516.6 TFLOP/s dense MFMA peak, with what limits
                 it in this run (its dQ atomics against their memory-side
                 rate, else the matrix cores);
  clock        : the gfx clock sampled with amdsmi while further untimed
                 steps of the same sweep run, and the MFMA peak at it;
  cpu_baseline : the fp64 CPU oracle timed on a bounded sample (c5 heads);
  dq_atomics   : the same kernel's 32-bit dQ accumulator atomics per launch
                 and their achieved rate over its launch time (these adds
                 execute at the memory side and bound the backward);
  per_config   : forward / backward times (mean, median, min over the timed
                 steps) and TFLOP/s per workload;
  memory_c3    : peak device memory of fused fwd+bwd vs an unfused S/P
                 PyTorch baseline at c3 (untimed pass);
  pages_sweep  : the pages' own forward speed comparison (standard fp16
                 attention vs the fused kernel, B=2 H=8 D=64 fp16 at
                 N = 2048/4096/8192, causal at 4096), untimed by the step;
  head_shard_c5_of_8 : one GPU's share of c5 split by heads over 8 GPUs
                 (B=1 H=2 N=16384 D=64 causal), forward + backward;
  fp8_forward  : the FP8 (E4M3) forward at the sweep's shapes against the
                 dense fp8 peak and the 16-bit forward, untimed by the step;
  split_kv     : the forward of short query blocks against a long key
                 history, whole key range per workgroup vs key splits;
  mha_layer    : forward + backward of the whole multi-head attention layer
                 (QKV projection, attention, output projection) with the
                 fused kernels against the same layer with standard fp16
                 attention, B=2 N=2048 embed 768, 12 heads, untimed by the
                 step.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2516.6  # MI355X dense bf16/fp16: 256 CU x 2.4 GHz x 4096 FLOP/clk
HBM_PEAK_TBPS = 8.0  # MI355X HBM3E, published
METRIC = "attention fwd+bwd TFLOPs/s and % of MFMA bf16 peak, N=512..16K, 1 GPU"
SWEEP = ("c2", "c3", "c4", "c5")
DOMINANT = "c5"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_bwd_dkdv_c5.json")


def conv_flops(w):
    f = 4.0 * w.B * w.H * w.N * w.N * w.D
    if w.causal:
        f /= 2
    return f, 2.5 * f


def dq_atomic_adds(w) -> int:
    """Number of 32-bit atomic adds one dK/dV launch issues into the dQ
    accumulator.  Each workgroup owns a block of 256 keys and adds its
    dS K contribution for every query row
    from the first one that sees its first key (causal) or from row 0, to
    the last row: D adds per row."""
    bkv = 256
    total = 0
    for kb0 in range(0, w.N, bkv):
        q_begin = kb0 if w.causal else 0
        total += (w.N - q_begin) * w.D
    return total * w.B * w.H


def kernel_source_hash() -> str:
    """Hash of the dK/dV kernel's sources, computed as the profiling harness
    computes it when it writes the traffic record (one definition)."""
    from io_aware_exact_02_amd.rocprof_harness import source_hash
    return source_hash()


def traffic_record():
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary, or None if absent or taken on different kernel code."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(budget_s: float):
    """The fp64 oracle (as it stands) on whole heads of c5, the workload that
    dominates the sweep, until the budget is used (at least one head);
    TFLOP/s under the same convention as the GPU figure."""
    from oracle import attention as oa
    from workloads import WORKLOADS, make_inputs
    w = WORKLOADS["c5"]
    inp = make_inputs(w)
    fwd_f, bwd_f = conv_flops(w)
    per_head = (fwd_f + bwd_f) / (w.B * w.H)
    done, t0 = 0, time.perf_counter()
    for h in range(w.H):
        sl = slice(h, h + 1)
        q, k, v, do = (inp[n][:, :, sl] for n in ("q", "k", "v", "do"))
        oa.attention_forward(q, k, v, causal=w.causal)
        oa.attention_backward(q, k, v, do, causal=w.causal)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(done * per_head / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": cpu_threads(), "kind": "oracle",
            "sample": f"fp64 numpy oracle, fwd+bwd of {done} of the {w.B * w.H} heads of c5 "
                      f"({w.describe()}), {dt:.1f} s; host {cpu_model()}, "
                      f"{len(os.sched_getaffinity(0))} cores in affinity"}


def unfused_memory_c3(torch, fa, w, inp):
    """Peak device memory of fused fwd+bwd vs the unfused three-step path
    (S = QK^T, P = softmax(S), O = PV, with S and P materialised) at c3."""
    dev = torch.device("cuda")
    qkv = inp["qkv"].to(dev)
    do = inp["do"].to(dev)
    torch.cuda.synchronize()
    res = {}
    # fused
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    q, k, v = qkv.unbind(dim=2)
    o, lse = fa.fwd(q, k, v, causal=False)
    dqkv = torch.empty_like(qkv)
    fa.bwd(q, k, v, o, lse, do, dq=dqkv[:, :, 0], dk=dqkv[:, :, 1], dv=dqkv[:, :, 2])
    torch.cuda.synchronize()
    res["fused_peak_bytes"] = torch.cuda.max_memory_allocated() - base
    del o, lse, dqkv
    # unfused: explicit products, contiguous operands only
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    scale = 1.0 / (w.D ** 0.5)
    qh, kh, vh = (t.permute(0, 2, 1, 3).contiguous() for t in qkv.unbind(dim=2))
    doh = do.permute(0, 2, 1, 3).contiguous()
    S = torch.matmul(qh, kh.transpose(-1, -2).contiguous()) * scale
    P = torch.softmax(S.float(), dim=-1).to(qkv.dtype)
    O = torch.matmul(P, vh)
    dV = torch.matmul(P.transpose(-1, -2).contiguous(), doh)
    dP = torch.matmul(doh, vh.transpose(-1, -2).contiguous())
    Dv = (doh.float() * O.float()).sum(-1, keepdim=True)
    dS = (P.float() * (dP.float() - Dv)).to(qkv.dtype)
    dQ = torch.matmul(dS, kh) * scale
    dK = torch.matmul(dS.transpose(-1, -2).contiguous(), qh) * scale
    torch.cuda.synchronize()
    res["unfused_peak_bytes"] = torch.cuda.max_memory_allocated() - base
    del S, P, O, dV, dP, Dv, dS, dQ, dK
    res["ratio"] = round(res["unfused_peak_bytes"] / max(res["fused_peak_bytes"], 1), 2)
    return res


def pages_sweep(torch, fa):
    """The speed comparison of the hotelren.com FlashAttention-2 walkthrough,
    section 4, on this GPU: forward time of the standard three-step attention
    (S = QK^T / sqrt(d), softmax, O = PV, all in fp16 with S and P
    materialised) against the fused kernel, the speedup, and the largest
    difference between the two outputs, for B=2, H=8, D=64 fp16 at N = 2048,
    4096, 8192; then the causal forward at N = 4096 against the non-causal
    one.  Also reported: each output's largest error against an fp32
    reference computed on the device."""
    from workloads import PAGES_SWEEP, make_inputs
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream(dev)

    def timed(fn, iters=10, warm=3):
        for _ in range(warm):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(iters):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / iters

    def standard(qt, kt, vt, causal, D, acc_dtype):
        # contiguous operands only; the mask is applied before the softmax
        attn = torch.matmul(qt.to(acc_dtype), kt.transpose(-2, -1).contiguous().to(acc_dtype))
        attn = attn / (D ** 0.5)
        if causal:
            n = attn.shape[-1]
            mask = torch.ones(n, n, dtype=torch.bool, device=dev).triu(1)
            attn = attn.masked_fill(mask, float("-inf"))
        attn = torch.softmax(attn, dim=-1)
        return torch.matmul(attn, vt.to(acc_dtype))

    rows = []
    fused_ms = {}
    for name, w in PAGES_SWEEP.items():
        inp = make_inputs(w)
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        qt, kt, vt = (t.transpose(1, 2).contiguous() for t in (q, k, v))
        t_std = timed(lambda: standard(qt, kt, vt, w.causal, w.D, q.dtype))
        t_fa = timed(lambda: fa.fwd(q, k, v, causal=w.causal))
        o_std = standard(qt, kt, vt, w.causal, w.D, q.dtype).transpose(1, 2).float()
        o_fa = fa.fwd(q, k, v, causal=w.causal)[0].float()
        o_ref = standard(qt, kt, vt, w.causal, w.D, torch.float32).transpose(1, 2)
        fused_ms[name] = t_fa
        rows.append({"seq_len": w.N, "causal": w.causal, "shape": w.describe(),
                     "standard_ms": round(t_std, 4), "fused_ms": round(t_fa, 4),
                     "speedup": round(t_std / t_fa, 2),
                     "max_err": float((o_std - o_fa).abs().max()),
                     "max_err_fp32_ref": {"standard": float((o_std - o_ref).abs().max()),
                                          "fused": float((o_fa - o_ref).abs().max())}})
        del q, k, v, qt, kt, vt, o_std, o_fa, o_ref
        torch.cuda.empty_cache()
    return {"rows": rows,
            "causal_vs_noncausal_fused_speedup_N4096": round(fused_ms["s4096"] / fused_ms["s4096c"], 2)}


PEAK_FP8_TFLOPS = 5033.2  # MI355X dense fp8 MFMA: twice the 16-bit rate


def fp8_forward(torch, fa, per_config):
    """The FP8 forward (E4M3 q, k, v with per-head descale factors, bf16
    output) at the shapes of the 16-bit sweep: time, TFLOP/s against the
    dense fp8 peak, and the speedup over the 16-bit forward measured in the
    same run.  Inputs: N(0,1) quantized per (batch, head), resident in HBM."""
    from workloads import WORKLOADS, fp8_random_inputs
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream(dev)
    rows = {}
    for name, cfg in per_config.items():
        if name not in WORKLOADS:  # profiling shapes: 16-bit only
            continue
        w = WORKLOADS[name]
        d = fp8_random_inputs(w.B, w.N, w.N, w.H, w.D, 9100 + w.N)
        q, k, v = (d[n].to(dev) for n in ("q", "k", "v"))
        ds = [d["descale_" + n].to(dev) for n in ("q", "k", "v")]
        o = torch.empty((w.B, w.N, w.H, w.D), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        run = lambda: fa.fwd_fp8(q, k, v, *ds, causal=w.causal, out=o, lse=lse)
        for _ in range(3):
            run()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(10):
            run()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / 10
        f = 4.0 * w.B * w.H * w.N * w.N * w.D / (2 if w.causal else 1)
        rows[name] = {"shape": f"B={w.B} H={w.H} N={w.N} D={w.D} e4m3 "
                               f"{'causal' if w.causal else 'non-causal'}",
                      "fwd_ms": round(ms, 4), "fwd_tflops": round(f / ms / 1e9, 2),
                      "pct_fp8_peak": round(100 * f / ms / 1e9 / PEAK_FP8_TFLOPS, 2),
                      "speedup_vs_16bit_fwd": round(cfg["fwd_ms"] / ms, 2)}
        del q, k, v, o, lse
    torch.cuda.empty_cache()
    return rows


def head_shard(torch, fa):
    """One GPU's share of c5 when its 16 heads are split over 8 GPUs (no
    exchange needed): B=1 H=2 N=16384 D=64 bf16 causal, forward + backward
    through the C ABI, 10 timed steps after 3 warm-ups.  128 workgroups in
    the backward; the forward splits the keys (fa_fwd_split_count's choice)
    because its 32-row waves alone would leave most of the device idle."""
    from workloads import Workload, make_inputs
    dev = torch.device("cuda")
    w = Workload("c5/8", 1, 2, 16384, 64, "bf16", True, "bnhd", 1005)
    inp = make_inputs(w)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, w.N), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(fa.workspace_bytes(1, 2, w.N, 64), dtype=torch.uint8, device=dev)

    def run():
        fa.fwd(q, k, v, causal=True, out=o, lse=lse)
        fa.bwd(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws)

    for _ in range(3):
        run()
    stream = torch.cuda.current_stream(dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(10):
        run()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / 10
    fwd_f, bwd_f = conv_flops(w)
    from io_aware_exact_02_amd import _lib
    splits = int(_lib.load().fa_fwd_split_count(1, 2, w.N, w.N, 64, 1))
    return {"shape": w.describe(), "fwd_key_splits": splits, "ms_per_step": round(ms, 4),
            "tflops": round((fwd_f + bwd_f) / ms / 1e9, 2),
            "pct_peak": round(100 * (fwd_f + bwd_f) / ms / 1e9 / PEAK_MFMA_TFLOPS, 2)}


def split_kv(torch, fa):
    """Forward of short query blocks against a long key history (one new row
    per head, a batch of them, or a 512-row chunk of a long context), causal
    mask aligned to the last key: the whole key range per workgroup
    (num_splits=1) against the key-split forward at fa_fwd_split_count's
    choice (partial results combined exactly by a second kernel).  One or two
    rows per head run the vector-unit kernel, more the tiled ones.  Each call
    goes straight to fa_fwd_split with a workspace allocated beforehand, so
    that the host's per-call work stays below the GPU time; 20 timed calls
    after 3 warm-ups each.  ``kv_gb_per_s`` is the K and V bytes of one call
    over the split time (these launches stream K and V once) and
    ``hbm_frac`` that rate over the 8 TB/s peak."""
    import ctypes
    from io_aware_exact_02_amd import _lib
    from workloads import random_qkv
    lib = _lib.load()
    dev = torch.device("cuda")
    shapes = [(1, 16, 1, 16384, 64), (8, 8, 1, 8192, 128), (64, 32, 1, 2048, 128),
              (1, 16, 512, 16384, 64)]

    def timed(fn, iters=20, warm=3):
        for _ in range(warm):
            fn()
        stream = torch.cuda.current_stream(dev)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(iters):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / iters

    rows = []
    for i, (B, H, Nq, Nk, D) in enumerate(shapes):
        qa = random_qkv(B, Nq, H, D, "bf16", 1200 + 2 * i)
        ka = random_qkv(B, Nk, H, D, "bf16", 1201 + 2 * i)
        q, k, v = qa["q"].to(dev), ka["k"].to(dev), ka["v"].to(dev)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
        S = int(lib.fa_fwd_split_count(B, H, Nq, Nk, D, 1))
        nbytes = int(lib.fa_fwd_split_workspace_bytes(B, H, Nq, D, S))
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        st = _lib.FwdStrides(*(_lib.Stride3(*t.stride()[:3]) for t in (q, k, v, o)))
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

        def call(splits):
            status = lib.fa_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                      lse.data_ptr(), B, H, Nq, Nk, D, 1, D ** -0.5,
                                      _lib.FA_BF16, ctypes.byref(st), splits, ws.data_ptr(),
                                      nbytes, stream)
            if status != _lib.FA_OK:
                raise RuntimeError(f"fa_fwd_split: status {status}")

        t1 = timed(lambda: call(1))
        ts = timed(lambda: call(S))
        kv_bytes = 2 * B * H * Nk * D * 2
        gbs = kv_bytes / ts / 1e6
        rows.append({"shape": f"B={B} H={H} Nq={Nq} Nk={Nk} D={D} bf16 causal",
                     "kernel": "vector-unit" if Nq <= 2 else "tiled",
                     "num_splits": S, "unsplit_ms": round(t1, 4), "split_ms": round(ts, 4),
                     "speedup": round(t1 / ts, 2), "kv_gb_per_s": round(gbs, 1),
                     "hbm_frac": round(gbs / (HBM_PEAK_TBPS * 1e3), 3)})
        del q, k, v, o, lse, ws
    torch.cuda.empty_cache()
    return rows


def mha_layer(torch, fa):
    """Training step of the multi-head attention layer (forward and backward
    of FlashMHA, random-init fp16 weights) at B=2, N=2048, embed 768, 12
    heads, against the same layer and weights with the attention step done
    the standard way (S and P materialised in fp16, autograd backward)."""
    dev = torch.device("cuda")
    B, N, E, H = 2, 2048, 768, 12
    D = E // H
    dt = torch.float16
    torch.manual_seed(7300)
    m = fa.FlashMHA(E, H, dtype=dt).to(dev)
    gen = torch.Generator("cpu").manual_seed(7301)
    x = torch.randn((B, N, E), generator=gen).to(dt).to(dev).requires_grad_(True)
    dy = torch.randn((B, N, E), generator=gen).to(dt).to(dev)
    stream = torch.cuda.current_stream(dev)

    def standard_layer():
        qkv = m.Wqkv(x).view(B, N, 3, H, D).permute(2, 0, 3, 1, 4)
        q, k, v = (t.contiguous() for t in qkv.unbind(0))
        s = torch.matmul(q, k.transpose(-2, -1).contiguous()) / (D ** 0.5)
        o = torch.matmul(torch.softmax(s, dim=-1), v)
        return m.out_proj(o.transpose(1, 2).reshape(B, N, E))

    def train_step(layer):
        m.zero_grad(set_to_none=True)
        x.grad = None
        layer().backward(dy)

    def timed(layer, iters=10, warm=3):
        for _ in range(warm):
            train_step(layer)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(iters):
            train_step(layer)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / iters

    t_fa = timed(lambda: m(x))
    t_std = timed(standard_layer)
    with torch.no_grad():
        diff = float((m(x).float() - standard_layer().float()).abs().max())
    del x, dy
    torch.cuda.empty_cache()
    return {"shape": f"B={B} N={N} embed={E} heads={H} head_dim={D} fp16 non-causal",
            "fused_ms": round(t_fa, 4), "standard_ms": round(t_std, 4),
            "speedup": round(t_std / t_fa, 2),
            "fused_tokens_per_s": round(B * N / (t_fa * 1e-3)),
            "max_output_diff": diff}


# Memory-side rate of 32-bit integer atomics measured with a throughput probe
# on MI355X: the ceiling of the dQ accumulation.  Used only when the probe
# program (built next to the library) cannot run; otherwise the rate is
# measured in the same run.
DQ_ATOMIC_PROBE_G_PER_S = 412.0
PROBE = os.path.join(ROOT, "io_aware_exact_02_amd", "atomic_probe")


def atomic_probe():
    """Run the atomic throughput probe (a child process on the same GPU,
    after the timed region): int32, paired-int64 and fp32 atomic adds in the
    dQ accumulation pattern of c5.  Returns its JSON, or None."""
    if not os.path.exists(PROBE):
        return None
    try:
        res = subprocess.run([PROBE], capture_output=True, text=True, timeout=120)
    except (OSError, subprocess.TimeoutExpired) as e:
        return {"error": str(e)}
    if res.returncode != 0:
        return {"error": (res.stdout + res.stderr)[-300:]}
    try:
        return json.loads(res.stdout.strip().splitlines()[-1])
    except (ValueError, IndexError):
        return {"error": res.stdout[-300:]}


def gfx_clock_sampler():
    """A start/stop pair that samples the GPU's gfx clock (MHz) through
    amdsmi in a background thread, or None when amdsmi is unavailable."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception:
        return None

    def read():
        try:
            m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
            for key in ("current_gfxclks", "current_gfxclk", "average_gfxclk_frequency"):
                v = m.get(key)
                if isinstance(v, (list, tuple)):
                    v = [x for x in v if isinstance(x, (int, float)) and 0 < x < 10000]
                    if v:
                        return float(statistics.mean(v))
                elif isinstance(v, (int, float)) and 0 < v < 10000:
                    return float(v)
        except Exception:
            pass
        try:
            info = amdsmi.amdsmi_get_clock_info(handle, amdsmi.AmdSmiClkType.GFX)
            v = info.get("clk")
            return float(v) if isinstance(v, (int, float)) and v > 0 else None
        except Exception:
            return None

    samples = []
    stop = threading.Event()

    def loop():
        while not stop.is_set():
            v = read()
            if v is not None:
                samples.append(v)
            time.sleep(0.005)

    th = threading.Thread(target=loop, daemon=True)

    def start():
        th.start()

    def finish():
        stop.set()
        th.join(timeout=2)
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass
        return samples

    return start, finish


def copy_calibration(torch, dev, mib):
    """One plain elementwise kernel that reads and writes `mib` MiB: what
    rocprofv3's FETCH_SIZE and WRITE_SIZE read for it scales theirs for the
    attention kernels."""
    if mib <= 0:
        return
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)  # one read + one write of n*4 bytes
    torch.cuda.synchronize()
    del src, dst


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # Defaults: 100 untimed steps bring the GPU to its sustained clock state
    # (runs with 5 warm-up steps measured about 5% lower, run after run), and
    # 200 timed steps take well under a second.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workloads", default=",".join(SWEEP))
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the CPU oracle baseline (0 = skip)")
    ap.add_argument("--no-memory", action="store_true", help="skip the c3 memory comparison")
    ap.add_argument("--no-pages-sweep", action="store_true",
                    help="skip the standard-vs-fused forward sweep of the pages (N=2048..8192)")
    ap.add_argument("--no-mha", action="store_true", help="skip the attention-layer measurement")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 forward measurement")
    ap.add_argument("--no-split", action="store_true",
                    help="skip the key-split forward measurement")
    ap.add_argument("--no-shard", action="store_true",
                    help="skip the one-GPU share of c5 under 8-way head sharding")
    ap.add_argument("--no-atomic-probe", dest="atomic_probe", action="store_false",
                    help="do not run the atomic throughput probe after the timed region")
    ap.add_argument("--clock-seconds", type=float, default=1.0,
                    help="after timing, run untimed sweep steps this long while sampling the "
                         "gfx clock (0 = skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run one plain elementwise kernel that reads and "
                         "writes this many MiB (calibrates HBM byte counters)")
    ap.add_argument("--only-split-kv", action="store_true",
                    help="run only the short-query / long-history forward measurement "
                         "(and the counter calibration) and print its rows as one JSON line")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the attention hot path here has no "
              "multi-GPU mode (heads shard across GPUs with no exchange); run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    import io_aware_exact_02_amd as fa
    from workloads import PROFILE_SHAPES, WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    if args.only_split_kv:
        rows = split_kv(torch, fa)
        copy_calibration(torch, dev, args.copy_calibration_mib)
        print(json.dumps({"split_kv": rows, "data": "synthetic"}), flush=True)
        return 0
    names = [n.strip() for n in args.workloads.split(",") if n.strip()]
    cases = []
    for name in names:
        w = WORKLOADS[name] if name in WORKLOADS else PROFILE_SHAPES[name]
        inp = make_inputs(w)
        c = {"w": w, "inp": inp}
        if w.layout == "packed":
            qkv = inp["qkv"].to(dev)
            c["q"], c["k"], c["v"] = qkv.unbind(dim=2)
            dqkv = torch.empty_like(qkv)
            c["dq"], c["dk"], c["dv"] = dqkv.unbind(dim=2)
            c["keep"] = (qkv, dqkv)
        else:
            c["q"], c["k"], c["v"] = (inp[n].to(dev) for n in ("q", "k", "v"))
            c["dq"], c["dk"], c["dv"] = (torch.empty_like(c["q"]) for _ in range(3))
        c["do"] = inp["do"].to(dev)
        c["o"] = torch.empty((w.B, w.N, w.H, w.D), dtype=w.torch_dtype, device=dev)
        c["lse"] = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        c["ws"] = torch.empty(fa.workspace_bytes(w.B, w.H, w.N, w.D), dtype=torch.uint8,
                              device=dev)
        c["fwd_f"], c["bwd_f"] = conv_flops(w)
        c["ev"] = []
        cases.append(c)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    def step(record):
        for c in cases:
            evs = {}
            if record:
                for key in ("f0", "f1", "k0", "k1", "b1"):
                    evs[key] = torch.cuda.Event(enable_timing=True)
                evs["f0"].record(stream)
            fa.fwd(c["q"], c["k"], c["v"], causal=c["w"].causal, out=c["o"], lse=c["lse"])
            if record:
                evs["f1"].record(stream)
            hook = (lambda tag, e=evs: e["k0" if tag == "dkdv_begin" else "k1"].record(stream)) \
                if record else None
            fa.bwd(c["q"], c["k"], c["v"], c["o"], c["lse"], c["do"], causal=c["w"].causal,
                   dq=c["dq"], dk=c["dk"], dv=c["dv"], workspace=c["ws"], stage_hook=hook)
            if record:
                evs["b1"].record(stream)
                c["ev"].append(evs)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step(True)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    flops_step = sum(c["fwd_f"] + c["bwd_f"] for c in cases)
    value = flops_step / (ms_per_step * 1e-3) / 1e12

    # The sustained clock under this load: untimed steps of the same sweep
    # right after the timed region, with amdsmi sampling the gfx clock.
    clock = None
    if args.clock_seconds > 0:
        sampler = gfx_clock_sampler()
        if sampler is not None:
            start_s, finish_s = sampler
            start_s()
            t_end = time.perf_counter() + args.clock_seconds
            while time.perf_counter() < t_end:
                for _ in range(5):
                    step(False)
                torch.cuda.synchronize()
            samples = finish_s()
            if samples:
                mhz = statistics.median(samples)
                clock = {"gfx_mhz_median": round(mhz, 1), "gfx_mhz_min": round(min(samples), 1),
                         "gfx_mhz_max": round(max(samples), 1), "samples": len(samples),
                         "source": f"amdsmi, {args.clock_seconds:g} s of untimed sweep steps "
                                   "after the timed region",
                         "mfma_peak_at_this_clock_tflops": round(
                             torch.cuda.get_device_properties(0).multi_processor_count
                             * mhz * 1e6 * 4096 / 1e12, 1)}

    probe = atomic_probe() if args.atomic_probe else None
    probe_rate = (probe or {}).get("i32_g_per_s")
    atomic_ceiling = probe_rate if probe_rate else DQ_ATOMIC_PROBE_G_PER_S

    per_config = {}
    for c in cases:
        w = c["w"]
        fwd_t = [e["f0"].elapsed_time(e["f1"]) for e in c["ev"]]
        bwd_t = [e["f1"].elapsed_time(e["b1"]) for e in c["ev"]]
        dkdv_t = [e["k0"].elapsed_time(e["k1"]) for e in c["ev"]]
        fwd_ms = sum(fwd_t) / len(fwd_t)
        bwd_ms = sum(bwd_t) / len(bwd_t)
        dkdv_ms = sum(dkdv_t) / len(dkdv_t)
        per_config[w.name] = {
            "shape": w.describe(),
            "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
            "bwd_dkdv_kernel_ms": round(dkdv_ms, 4),
            "dq_atomic_adds": dq_atomic_adds(w),
            "dq_atomic_g_per_s": round(dq_atomic_adds(w) / dkdv_ms / 1e6, 1),
            "fwd_tflops": round(c["fwd_f"] / fwd_ms / 1e9, 2),
            "bwd_tflops": round(c["bwd_f"] / bwd_ms / 1e9, 2),
            "fwd_pct_peak": round(100 * c["fwd_f"] / fwd_ms / 1e9 / PEAK_MFMA_TFLOPS, 2),
            "bwd_pct_peak": round(100 * c["bwd_f"] / bwd_ms / 1e9 / PEAK_MFMA_TFLOPS, 2),
            # Per-launch statistics of the same event pairs (the means above
            # include every timed step).
            "fwd_ms_median": round(statistics.median(fwd_t), 4), "fwd_ms_min": round(min(fwd_t), 4),
            "bwd_ms_median": round(statistics.median(bwd_t), 4), "bwd_ms_min": round(min(bwd_t), 4),
            "bwd_dkdv_kernel_ms_median": round(statistics.median(dkdv_t), 4),
            "bwd_dkdv_kernel_ms_min": round(min(dkdv_t), 4),
            "fwd_pct_peak_at_median": round(
                100 * c["fwd_f"] / statistics.median(fwd_t) / 1e9 / PEAK_MFMA_TFLOPS, 2),
            "bwd_pct_peak_at_median": round(
                100 * c["bwd_f"] / statistics.median(bwd_t) / 1e9 / PEAK_MFMA_TFLOPS, 2),
        }

    roofline = None
    atomics = None
    dom = next((c for c in cases if c["w"].name == DOMINANT), None)
    if dom is not None:
        dkdv_ms = per_config[DOMINANT]["bwd_dkdv_kernel_ms"]
        achieved = dom["bwd_f"] / dkdv_ms / 1e9
        adds = dq_atomic_adds(dom["w"])
        rate = adds / dkdv_ms / 1e6
        # What limits the kernel, from this run's numbers: its dQ atomics
        # against the memory-side atomic rate, else the matrix cores.
        limiter = ("dq atomics (memory-side)" if rate >= 0.8 * atomic_ceiling
                   else "matrix cores / latency")
        roofline = {"bound": "mfma", "kernel": "bwd_dkdv_kernel",
                    "workload": dom["w"].describe(),
                    "flops_per_launch": dom["bwd_f"],
                    "avg_launch_ms": dkdv_ms,
                    "achieved": round(achieved, 2), "peak": PEAK_MFMA_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_TFLOPS, 4),
                    "traffic": traffic_record(),
                    "limited_by": {"what": limiter,
                                   "dq_atomic_g_per_s": round(rate, 1),
                                   "atomic_probe_g_per_s": round(atomic_ceiling, 1),
                                   "atomic_probe": probe if probe else
                                   {"fixed_g_per_s": DQ_ATOMIC_PROBE_G_PER_S},
                                   "frac_of_atomic_rate": round(rate / atomic_ceiling, 3)}}
        atomics = {"kernel": "bwd_dkdv_kernel", "workload": dom["w"].describe(),
                   "adds_per_launch": adds, "bytes_per_add": 4,
                   "avg_launch_ms": dkdv_ms,
                   "achieved_g_adds_per_s": round(adds / dkdv_ms / 1e6, 1),
                   "achieved_payload_tb_per_s": round(4 * adds / dkdv_ms / 1e9, 3)}

    copy_calibration(torch, dev, args.copy_calibration_mib)

    memory = None
    if not args.no_memory and "c3" in names:
        c3 = next(c for c in cases if c["w"].name == "c3")
        memory = unfused_memory_c3(torch, fa, c3["w"], c3["inp"])

    sweep = None
    if not args.no_pages_sweep:
        sweep = pages_sweep(torch, fa)

    shard = None
    if not args.no_shard:
        shard = head_shard(torch, fa)

    fp8 = None
    if not args.no_fp8:
        fp8 = fp8_forward(torch, fa, per_config)

    splits = None
    if not args.no_split:
        splits = split_kv(torch, fa)

    layer = None
    if not args.no_mha:
        layer = mha_layer(torch, fa)

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(args.cpu_seconds)

    dtypes = sorted({c["w"].dtype for c in cases})
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "wall_s_timed": round(wall, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "+".join(dtypes) + " (fp32 accumulate)",
        "data": "synthetic: seeded N(0,1) q, k, v, dO",
        "config": {"workload": "attention fwd+bwd sweep " + ", ".join(
            f"{c['w'].name}: {c['w'].describe()}" for c in cases),
            "flops_per_step": flops_step},
        "pct_of_peak": round(100 * value / PEAK_MFMA_TFLOPS, 2),
        "clock": clock,
        "roofline": roofline,
        "dq_atomics": atomics,
        "cpu_baseline": cpu,
        "per_config": per_config,
        "memory_c3": memory,
        "pages_sweep": sweep,
        "mha_layer": layer,
        "fp8_forward": fp8,
        "head_shard_c5_of_8": shard,
        "split_kv": splits,
        # The marketing name can be empty where libdrm's amdgpu.ids table is
        # not installed; the architecture name is always there.
        "device": {"name": torch.cuda.get_device_properties(0).name
                   or getattr(torch.cuda.get_device_properties(0), "gcnArchName", ""),
                   "compute_units": torch.cuda.get_device_properties(0).multi_processor_count,
                   "derived_peak_tflops": round(
                       torch.cuda.get_device_properties(0).multi_processor_count
                       * 2.4e9 * 4096 / 1e12, 1),
                   "clock_for_peak_ghz": 2.4},
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

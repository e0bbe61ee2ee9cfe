"""rocprofv3 harness: kernel times, MFMA utilisation and HBM traffic of the
attention kernels, measured on ``bench.py``.

    python -m io_aware_exact_02_amd.rocprof_harness --raw /tmp/prof \\
        [--workloads c2,c3,c4,c5] [--summary-dir profiles]

(``--workloads split_kv`` profiles bench.py's short-query / long-history
forwards instead: ``bench.py --only-split-kv``.)

Four rocprofv3 runs of ``bench.py`` (each its own process; counters never
share a run with tracing):

1. ``--kernel-trace --stats``: per-kernel dispatch count and durations;
2. ``--pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F16
   SQ_INSTS_VALU_MFMA_MOPS_F8``: executed matrix-core FLOPs (512 FLOPs per
   MOPS unit), per dispatch;
3. ``--pmc FETCH_SIZE`` and 4. ``--pmc WRITE_SIZE``: bytes between L2 and
   memory (KiB per dispatch), each calibrated against one elementwise kernel
   of known size (one read and one write of ``--calib-mib`` MiB) run in the
   same process;
5. ``--kernel-trace --pmc`` of GRBM_GUI_ACTIVE and seven SQ counters: the
   clock, matrix-core and VALU busy fractions, the share of wave cycles
   spent waiting, and LDS activity and bank conflicts per kernel, written to
   ``utilization_<workloads>.txt``.

It prints the summary and, with ``--summary-dir``, writes
``kernels_<workloads>.txt`` (durations, executed MFMA TFLOP/s against the
dense peak of the kernel's type -- 2516.6 TFLOP/s bf16/fp16, 5033.2 TFLOP/s
fp8 -- and L2-to-memory GB/s) and, when c5 is
profiled, ``traffic_bwd_dkdv_c5.json`` -- the calibrated bytes per launch of
the dK/dV kernel together with a hash of its sources, which ``bench.py``
reports as the roofline's ``traffic`` while the sources are unchanged.
This module never touches the GPU itself; only its rocprofv3 children do.
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")
PEAK_TFLOPS = 2516.6
PEAK_FP8_TFLOPS = 5033.2
KERNEL_SOURCES = [os.path.join(ROOT, "io_aware_exact_02_amd", "csrc", f)
                  for f in ("fa_bwd.hip", "fa_device.hpp", "fa_kernels.hpp", "fa_xcd.hpp")]


def source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def grid_size(r) -> str:
    """Total work-items of a dispatch (counter CSV: Grid_Size; trace CSV:
    Grid_Size_X/Y/Z)."""
    if "Grid_Size" in r:
        return r["Grid_Size"]
    return str(int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]))


def short_name(kernel: str) -> str:
    k = kernel.replace("void ", "").replace("(anonymous namespace)::", "").replace("fa::", "")
    return k.split("(")[0].strip()


def run(cmd, timeout, log):
    print("+", " ".join(cmd), flush=True)
    with open(log, "w") as f:
        proc = subprocess.run(cmd, stdout=f, stderr=subprocess.STDOUT, timeout=timeout)
    if proc.returncode != 0:
        with open(log) as f:
            tail = f.read()[-2000:]
        raise RuntimeError(f"exit {proc.returncode}: {' '.join(cmd)}\n{tail}")


def bench_cmd(workloads, steps, warmup, calib_mib):
    if workloads == "split_kv":
        # The short-query / long-history forwards alone (bench.py split_kv).
        return [sys.executable, BENCH, "--only-split-kv", "--copy-calibration-mib",
                str(calib_mib)]
    return [sys.executable, BENCH, "--steps", str(steps), "--warmup", str(warmup), "--cpu-seconds", "0",
            "--no-memory", "--no-pages-sweep", "--no-mha", "--no-shard", "--no-split",
            # No kernels after the timed region: the summary's "timed" column
            # takes each kernel's last dispatches.
            "--clock-seconds", "0", "--no-atomic-probe",
            "--workloads", workloads,
            "--copy-calibration-mib", str(calib_mib)]


def rocprof(args, out, bench):
    return ["rocprofv3", *args, "--output-format", "csv", "-d", out, "-o", "run", "--", *bench]


def read_csv(pattern):
    files = glob.glob(pattern, recursive=True)
    if not files:
        raise RuntimeError(f"no rocprofv3 output matches {pattern}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


UTIL_COUNTERS = ["GRBM_GUI_ACTIVE", "SQ_WAVE_CYCLES", "SQ_BUSY_CU_CYCLES",
                 "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_WAIT_ANY",
                 "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT"]
XCDS, CUS, SIMDS = 8, 256, 1024


def timed_counters(rows, steps):
    """kernel -> {counter: mean over the kernel's last `steps` dispatches}.
    Counter values are summed over all hardware instances (GRBM_GUI_ACTIVE
    over the 8 XCDs, SQ counters over all CUs or SIMDs)."""
    per = collections.defaultdict(lambda: collections.defaultdict(dict))
    for r in rows:
        k = short_name(r["Kernel_Name"]) + f" grid={grid_size(r)}"
        per[k][r["Counter_Name"]][int(r["Dispatch_Id"])] = float(r["Counter_Value"])
    out = {}
    for k, d in per.items():
        out[k] = {}
        for c, v in d.items():
            vals = [v[i] for i in sorted(v)][-steps:]
            out[k][c] = sum(vals) / len(vals)
    return out


def utilization_lines(rows, trace_rows, steps, kernels):
    """Per kernel, from one --kernel-trace --pmc run (rocprof's derived-metric
    formulas): clock = XCD cycles / duration; MFMA busy = MFMA busy cycles /
    (SIMDs x cycles); VALU busy = 4 x VALU-active quad cycles / (SIMDs x
    cycles); waiting = wave cycles waiting on anything / all wave cycles; LDS
    active = LDS-index-active cycles / (CUs x cycles); bank conflicts as a
    share of LDS-active cycles."""
    ctr = timed_counters(rows, steps)
    dur = collections.defaultdict(list)
    for r in sorted(trace_rows, key=lambda r: int(r["Start_Timestamp"])):
        k = short_name(r["Kernel_Name"]) + f" grid={grid_size(r)}"
        dur[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    lines = [f"{'kernel (grid)':64s} {'us':>8s} {'GHz':>5s} {'MFMA%':>6s} {'VALU%':>6s} "
             f"{'wait%':>6s} {'LDS%':>6s} {'bank%':>6s}"]
    for k in kernels:
        c = ctr.get(k)
        d = dur.get(k)
        if not c or not d or not c.get("GRBM_GUI_ACTIVE"):
            continue
        t = sum(d[-steps:]) / len(d[-steps:])
        cyc = c["GRBM_GUI_ACTIVE"] / XCDS
        pct = lambda x: 100.0 * x
        lines.append(
            f"{k[:64]:64s} {t * 1e6:8.1f} {cyc / t / 1e9:5.2f} "
            f"{pct(c.get('SQ_VALU_MFMA_BUSY_CYCLES', 0) / (SIMDS * cyc)):6.1f} "
            f"{pct(4 * c.get('SQ_ACTIVE_INST_VALU', 0) / (SIMDS * cyc)):6.1f} "
            f"{pct(c.get('SQ_WAIT_ANY', 0) / max(c.get('SQ_WAVE_CYCLES', 0), 1)):6.1f} "
            f"{pct(c.get('SQ_LDS_IDX_ACTIVE', 0) / (CUS * cyc)):6.1f} "
            f"{pct(c.get('SQ_LDS_BANK_CONFLICT', 0) / max(c.get('SQ_LDS_IDX_ACTIVE', 0), 1)):6.1f}")
    return lines


def counters_by_kernel(rows):
    """kernel -> {counter: [value per dispatch]}"""
    per = collections.defaultdict(lambda: collections.defaultdict(dict))
    for r in rows:
        k = short_name(r["Kernel_Name"]) + f" grid={grid_size(r)}"
        per[k][r["Counter_Name"]][r["Dispatch_Id"]] = float(r["Counter_Value"])
    return {k: {c: list(v.values()) for c, v in d.items()} for k, d in per.items()}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--raw", required=True, help="directory for raw rocprofv3 output")
    ap.add_argument("--workloads", default="c2,c3,c4,c5")
    # The bench's own timed region: its average then matches the bench's events.
    ap.add_argument("--steps", type=int, default=200)
    # The same warm-up as bench.py's default: the GPU reaches its sustained
    # clock state only after about a hundred steps.
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--calib-mib", type=int, default=512)
    ap.add_argument("--summary-dir", default=None)
    ap.add_argument("--timeout", type=int, default=300)
    ap.add_argument("--summarize-only", action="store_true",
                    help="re-read the raw output of an earlier run instead of profiling")
    a = ap.parse_args(argv)
    os.makedirs(a.raw, exist_ok=True)
    bench = bench_cmd(a.workloads, a.steps, a.warmup, a.calib_mib)

    t0 = time.time()
    if not a.summarize_only:
        run(rocprof(["--kernel-trace", "--stats"], os.path.join(a.raw, "trace"), bench),
            a.timeout, os.path.join(a.raw, "trace.log"))
    stats = read_csv(os.path.join(a.raw, "trace", "**", "*kernel_stats.csv"))
    trace = read_csv(os.path.join(a.raw, "trace", "**", "*kernel_trace.csv"))
    passes = {
        "mfma": ["SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16",
                 "SQ_INSTS_VALU_MFMA_MOPS_F8"],
        "fetch": ["FETCH_SIZE"],
        "write": ["WRITE_SIZE"],
    }
    ctr = {}
    for name, cs in passes.items():
        out = os.path.join(a.raw, f"pmc_{name}")
        if not a.summarize_only:
            run(rocprof(["--pmc", *cs], out, bench), a.timeout,
                os.path.join(a.raw, f"pmc_{name}.log"))
        ctr[name] = counters_by_kernel(read_csv(os.path.join(out, "**", "*counter_collection.csv")))

    util_out = os.path.join(a.raw, "pmc_util")
    if not a.summarize_only:
        run(rocprof(["--kernel-trace", "--pmc", *UTIL_COUNTERS], util_out, bench), a.timeout,
            os.path.join(a.raw, "pmc_util.log"))
    util_rows = read_csv(os.path.join(util_out, "**", "*counter_collection.csv"))
    util_trace = read_csv(os.path.join(util_out, "**", "*kernel_trace.csv"))

    # Durations per (kernel, grid) from the trace, in dispatch order.  The
    # bench launches each sweep kernel warmup + steps times; "timed" is the
    # mean over the last `steps` dispatches, the ones bench.py times.
    dur = collections.defaultdict(list)
    for r in sorted(trace, key=lambda r: int(r["Start_Timestamp"])):
        k = short_name(r["Kernel_Name"]) + f" grid={grid_size(r)}"
        dur[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)

    def timed_avg(d):
        tail = d[-a.steps:] if len(d) >= a.steps else d
        return sum(tail) / len(tail)

    # Calibration: the elementwise kernel moves calib_mib MiB each way.
    calib = [k for k in ctr["fetch"] if "neg" in k.lower()]
    expect_kib = a.calib_mib * 1024.0
    f_scale = w_scale = None
    if calib:
        f_meas = sum(ctr["fetch"][calib[0]]["FETCH_SIZE"]) / len(ctr["fetch"][calib[0]]["FETCH_SIZE"])
        wk = [k for k in ctr["write"] if "neg" in k.lower()][0]
        w_meas = sum(ctr["write"][wk]["WRITE_SIZE"]) / len(ctr["write"][wk]["WRITE_SIZE"])
        f_scale, w_scale = expect_kib / f_meas, expect_kib / w_meas

    lines = [f"rocprofv3 summary of bench.py --workloads {a.workloads} "
             f"(steps {a.steps}, warmup {a.warmup})",
             "command: python -m io_aware_exact_02_amd.rocprof_harness --raw <dir> "
             f"--workloads {a.workloads} --steps {a.steps} --warmup {a.warmup} --calib-mib {a.calib_mib}",
             "  runs: rocprofv3 --kernel-trace --stats --output-format csv -- python3 bench.py "
             + " ".join(bench[2:]),
             "        and the same command under rocprofv3 --pmc "
             + " ".join(passes["mfma"]) + " / --pmc FETCH_SIZE / --pmc WRITE_SIZE",
             f"calibration: elementwise kernel of {a.calib_mib} MiB read + write; counter scale "
             f"FETCH x{f_scale:.4f}, WRITE x{w_scale:.4f}" if f_scale else "calibration: none",
             "",
             f"{'kernel (grid)':64s} {'calls':>5s} {'avg us':>9s} {'timed us':>9s} {'min us':>9s} "
             f"{'MFMA TF/s':>9s} {'%peak':>6s} {'rd GB/s':>8s} {'wr GB/s':>8s}"]
    record = None
    for k in sorted(dur, key=lambda x: -sum(dur[x])):
        d = dur[k]
        avg = sum(d) / len(d)
        mf = ctr["mfma"].get(k, {})
        mops = 0.0
        for c in passes["mfma"]:
            if c in mf:
                mops += sum(mf[c]) / len(mf[c])
        flops = mops * 512
        fe = ctr["fetch"].get(k, {}).get("FETCH_SIZE")
        wr = ctr["write"].get(k, {}).get("WRITE_SIZE")
        rd_b = (sum(fe) / len(fe)) * 1024 * (f_scale or 1.0) if fe else None
        wr_b = (sum(wr) / len(wr)) * 1024 * (w_scale or 1.0) if wr else None
        tf = flops / avg / 1e12 if avg > 0 else 0.0
        peak = PEAK_FP8_TFLOPS if "fwd8" in k else PEAK_TFLOPS
        lines.append(f"{k[:64]:64s} {len(d):5d} {avg * 1e6:9.1f} {timed_avg(d) * 1e6:9.1f} "
                     f"{min(d) * 1e6:9.1f} "
                     f"{tf:9.1f} {100 * tf / peak:6.1f} "
                     f"{(rd_b / avg / 1e9) if rd_b else 0:8.1f} {(wr_b / avg / 1e9) if wr_b else 0:8.1f}")
        # The dominant kernel: the bf16 head_dim-64 causal dK/dV kernel (only
        # c5 launches it), the longest-running entry of that name.
        if ("c5" in a.workloads.split(",") and record is None and "bwd_dkdv_kernel" in k
                and "BF16, 64" in k and "true" in k):
            record = {"kernel": k, "workload": "c5: B=1 H=16 N=16384 D=64 bf16 causal",
                      "avg_launch_us": avg * 1e6,
                      "timed_avg_launch_us": timed_avg(d) * 1e6,
                      "fetch_bytes_per_launch": rd_b, "write_bytes_per_launch": wr_b,
                      "hbm_bytes_per_launch": (rd_b or 0) + (wr_b or 0),
                      "executed_mfma_flops_per_launch": flops,
                      "calibration": {"mib": a.calib_mib, "fetch_scale": f_scale,
                                      "write_scale": w_scale},
                      "kernel_source_hash": source_hash()}
    lines.append("")
    lines.append("kernel stats (rocprofv3 --stats):")
    try:
        for r in sorted(stats, key=lambda r: -float(r.get("TotalDurationNs", 0)))[:12]:
            lines.append(f"  {short_name(r['Name'])[:70]:70s} calls {r['Calls']:>5s} "
                         f"avg {float(r['AverageNs']) / 1e3:9.1f} us  "
                         f"total {float(r['TotalDurationNs']) / 1e6:8.3f} ms  "
                         f"{float(r['Percentage']):5.1f}%")
    except (KeyError, ValueError):
        lines.append("  (unexpected kernel_stats.csv columns: "
                     f"{sorted(stats[0].keys()) if stats else []})")
    text = "\n".join(lines)
    print(text)
    sweep = [k for k in sorted(dur, key=lambda x: -sum(dur[x])) if "neg" not in k.lower()][:10]
    util = "\n".join([
        f"rocprofv3 utilization of bench.py --workloads {a.workloads} (steps {a.steps}, "
        f"warmup {a.warmup}; means over each kernel's last {a.steps} dispatches)",
        "command: python -m io_aware_exact_02_amd.rocprof_harness --raw <dir> "
        f"--workloads {a.workloads} --steps {a.steps} --warmup {a.warmup} --calib-mib {a.calib_mib}",
        "  run: rocprofv3 --kernel-trace --pmc " + " ".join(UTIL_COUNTERS)
        + " --output-format csv -- python3 bench.py " + " ".join(bench[2:]),
        "", *utilization_lines(util_rows, util_trace, a.steps, sweep)])
    print(util)
    print(f"[harness] {time.time() - t0:.0f} s", flush=True)
    if a.summary_dir:
        os.makedirs(a.summary_dir, exist_ok=True)
        tag = a.workloads.replace(",", "-")
        with open(os.path.join(a.summary_dir, f"kernels_{tag}.txt"), "w") as f:
            f.write(text + "\n")
        with open(os.path.join(a.summary_dir, f"utilization_{tag}.txt"), "w") as f:
            f.write(util + "\n")
        if record is not None:
            with open(os.path.join(a.summary_dir, "traffic_bwd_dkdv_c5.json"), "w") as f:
                json.dump(record, f, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Host-side checks of bench.py (no GPU): the FLOP convention, the dQ
atomic count it divides by, the one-GPU rule and the traffic record's
guard against stale counter data."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import WORKLOADS, Workload  # noqa: E402


@pytest.mark.parametrize("name,fwd_gflop", [("c2", 1.610612736), ("c3", 25.769803776),
                                            ("c4", 137.438953472), ("c5", 549.755813888)])
def test_flop_convention(name, fwd_gflop):
    """4 B H N^2 D for the two products of the forward, halved when causal;
    the backward counts 2.5 times the forward (five products against two).
    Expected values written out from those closed forms for each shape."""
    fwd, bwd = bench.conv_flops(WORKLOADS[name])
    assert fwd == pytest.approx(fwd_gflop * 1e9, rel=1e-12)
    assert bwd == pytest.approx(2.5 * fwd_gflop * 1e9, rel=1e-12)


def _atomics_by_rows(w):
    """Count row by row: a query row r takes D atomic adds from every key
    block whose first key it sees (causal: first key <= r; otherwise every
    block), the dQ elements of that row."""
    bkv = 256
    blocks = (w.N + bkv - 1) // bkv
    total = 0
    for r in range(w.N):
        seen = min(r // bkv + 1, blocks) if w.causal else blocks
        total += seen * w.D
    return total * w.B * w.H


@pytest.mark.parametrize("w", [
    WORKLOADS["c3"], WORKLOADS["c4"], WORKLOADS["c5"],
    Workload("adhoc", 2, 3, 1000, 64, "bf16", True, "bnhd", 0),
    Workload("adhoc", 1, 2, 1000, 128, "f16", False, "bnhd", 0),
    Workload("adhoc", 1, 1, 129, 128, "bf16", True, "bnhd", 0),
], ids=["c3", "c4", "c5", "ragged-causal-64", "ragged-128", "short-causal-128"])
def test_dq_atomic_count(w):
    assert bench.dq_atomic_adds(w) == _atomics_by_rows(w)


def test_dq_atomic_count_values():
    """The counts quoted for the two causal sweep workloads."""
    assert bench.dq_atomic_adds(WORKLOADS["c5"]) == 545_259_520
    assert bench.dq_atomic_adds(WORKLOADS["c4"]) == 138_412_032


def test_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr


def test_traffic_record_guard(tmp_path, monkeypatch):
    """The counter record is used only while the kernel sources hash to the
    value stored with it."""
    rec = {"hbm_bytes_per_launch": 1234.0, "kernel_source_hash": bench.kernel_source_hash()}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.traffic_record() == 1234.0
    rec["kernel_source_hash"] = "0" * 16
    path.write_text(json.dumps(rec))
    assert bench.traffic_record() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic_record() is None

"""CPU checks of the workgroup -> (head, item) mapping the forward, FP8
forward and backward kernels use to keep each head's workgroups on few XCDs
(each XCD has its own L2; workgroup id i runs on XCD i % 8).

The header is compiled host-only into tests/xcd_map_check.cpp, which checks
every B*H in 1..96 and item count in 1..80: each (head, item) pair is named
by exactly one id, items reach each XCD window by window, the heads per XCD
and XCDs per head stay within their bounds, and the work per XCD balances.
The dumped mappings below pin the cases by hand.
"""

import os
import shutil
import subprocess
from collections import defaultdict

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "io_aware_exact_02_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    out = str(tmp_path_factory.mktemp("xcd") / "xcd_map_check")
    subprocess.run([HIPCC, "-x", "hip", "--offload-host-only", "-O1", "-I", CSRC,
                    os.path.join(ROOT, "tests", "xcd_map_check.cpp"), "-o", out],
                   check=True, capture_output=True, timeout=300)
    return out


def dump(checker, BH, R):
    txt = subprocess.run([checker, "dump", str(BH), str(R)], check=True,
                         capture_output=True, text=True, timeout=60).stdout
    return [tuple(int(v) for v in line.split()) for line in txt.splitlines()]


def test_exhaustive(checker):
    r = subprocess.run([checker, "check"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok "), r.stdout + r.stderr


def test_twelve_heads_two_per_xcd(checker):
    """B*H = 12, 64 items: i % 12 puts three heads on each XCD; the mapping
    puts two, each head on one or two XCDs, 96 items per XCD."""
    rows = dump(checker, 12, 64)
    heads, count = defaultdict(set), defaultdict(int)
    for _, x, bh, item, valid in rows:
        assert valid
        heads[x].add(bh)
        count[x] += 1
    assert all(len(heads[x]) == 2 for x in range(8)), dict(heads)
    assert all(count[x] == 96 for x in range(8))
    old = defaultdict(set)
    for i in range(12 * 64):
        old[i % 8].add(i % 12)
    assert all(len(old[x]) == 3 for x in range(8))


def test_two_heads_match_plain_mapping(checker):
    """B*H = 2 (and any divisor or multiple of 8): bh = i % BH, item = i / BH;
    head 0 on the even XCDs, head 1 on the odd ones."""
    for BH, R in ((2, 64), (1, 9), (4, 7), (16, 5), (24, 3)):
        rows = dump(checker, BH, R)
        valid = [(i, bh, item) for i, _, bh, item, v in rows if v]
        assert len(valid) == BH * R
        assert all(bh == i % BH and item == i // BH for i, bh, item in valid), (BH, R)


def test_three_heads_ragged_last_window(checker):
    """B*H = 3 (one group of 3 heads over 8 XCDs), R = 5: one window of 8
    items per head pair, ids past item 4 name nothing and are marked so."""
    rows = dump(checker, 3, 5)
    assert len(rows) == 8 * 3 * 1
    valid = [(bh, item) for _, _, bh, item, v in rows if v]
    assert sorted(valid) == [(h, r) for h in range(3) for r in range(5)]
    for _, _, bh, item, v in rows:
        assert v == (item < 5)

"""The LDS-poisoning debug build really poisons (CPU).

tests/test_race_detection.py trusts libfa_poison.so to fill every LDS array
with NaN bits before a workgroup's first barrier.  Here the FP8 forward
kernels are compiled to gfx950 assembly with and without FA_POISON_LDS: in
the poisoned form each kernel stores all-ones words to LDS before its first
barrier (one store loop per LDS array), in the normal form it stores
nothing to LDS before that barrier.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "io_aware_exact_02_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _stores_before_first_barrier(asm: str):
    """Per kernel: (LDS stores, moves of -1) before its first s_barrier."""
    out = []
    for body in re.split(r"\n_Z\S*fwd8_kernel\S*:", asm)[1:]:
        head = body.split("s_barrier", 1)[0]
        out.append((len(re.findall(r"\bds_write", head)),
                    len(re.findall(r"v_mov_b32\S*\s+v\d+, -1\s*$", head, re.M))))
    return out


@pytest.mark.parametrize("poison", [0, 1])
def test_poison_fill_in_assembly(tmp_path, poison):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    out = str(tmp_path / "fwd8.s")
    subprocess.run([HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only",
                    "-S", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    f"-DFA_POISON_LDS={poison}", os.path.join(CSRC, "fa_fwd8.hip"), "-o", out],
                   check=True, capture_output=True, timeout=600)
    with open(out) as f:
        kernels = _stores_before_first_barrier(f.read())
    assert len(kernels) >= 4, kernels
    for stores, ones in kernels:
        if poison:
            # Ks0, Ks1, Vs0, Vs1 and the merge scratch: a store loop each.
            assert stores >= 5 and ones >= 5, kernels
        else:
            assert stores == 0 and ones == 0, kernels

"""The C ABI's host side under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU).

fa_api.cpp -- argument validation, workspace layout, stream and launch
handling -- is recompiled with both sanitizers on its host half and linked,
with the kernel objects of the normal build, into the C++ program
tests/host_sanitize_check.cpp, which calls every entry point of
include/fa.h with invalid arguments (each must return its status code) and,
with no GPU visible, with well-formed ones (FA_ERR_HIP).  A sanitizer
report, or any status other than the documented one, fails the test.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "io_aware_exact_02_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
from io_aware_exact_02_amd import build as _build  # noqa: E402  (source list only)

OBJS = [os.path.join(ROOT, "_build", f.rsplit(".", 1)[0] + ".o")
        for f in _build.SOURCES if f != "fa_api.cpp"]
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# Sanitizers on the host half only (the device half is never sanitized).
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


@pytest.mark.skipif(not all(os.path.exists(o) for o in OBJS),
                    reason="kernel objects not built (python -m io_aware_exact_02_amd.build)")
def test_abi_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    api = str(tmp_path / "fa_api.o")
    chk = str(tmp_path / "check.o")
    exe = str(tmp_path / "host_sanitize_check")
    run = lambda cmd: subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=600)
    run([HIPCC, "-x", "hip", "-std=c++17", "-O1", "-g", "-fPIC", "--offload-arch=gfx950",
         *SAN, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, "fa_api.cpp"), "-o", api])
    run([HIPCC, "-x", "hip", "--offload-host-only", "-std=c++17", "-g", *SAN, "-I", INCLUDE,
         "-c", os.path.join(ROOT, "tests", "host_sanitize_check.cpp"), "-o", chk])
    run([HIPCC, "--offload-arch=gfx950", *SAN, chk, api, *OBJS, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = res.stdout + res.stderr
    assert res.returncode == 0 and "ok " in res.stdout, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out

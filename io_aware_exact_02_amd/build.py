"""Build libfa.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m io_aware_exact_02_amd.build [--verbose]

Each source is compiled by hipcc into an object under ``_build/`` and the
objects are linked into ``io_aware_exact_02_amd/libfa.so`` next to this file;
a second build with LDS poisoning goes to ``libfa_poison.so`` (tests only),
and the atomic throughput probe that bench.py runs to ``atomic_probe``.
Always recompiles (the build check must exercise the compiler every time).
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
POISON_LIB = os.path.join(PKG, "libfa_poison.so")
PROBE = os.path.join(PKG, "atomic_probe")

SOURCES = ["fa_fwd.hip", "fa_fwd64.hip", "fa_fwd8.hip", "fa_decode.hip", "fa_bwd.hip", "fa_merge.hip",
           "fa_api.cpp"]
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled: hipcc would otherwise fuse scalar
# float math into v_pk_* instructions.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP toolchain is required to build libfa")
    return path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n"
                           f"{res.stdout}\n{res.stderr}")
    # hipcc's host pass does not know the packed-fp32 feature; drop that note.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(x for x in res.stderr.splitlines() if noise not in x and x.strip())
    if verbose and err:
        print(err, file=sys.stderr)
    return res


def build(verbose: bool = False, extra_flags=(), poison: bool = False) -> str:
    """Compile every source and link libfa.so; returns the library path.

    ``poison=True`` builds libfa_poison.so instead: the same kernels with
    every LDS array filled with NaN bits when a workgroup starts
    (FA_POISON_LDS), for the tests that look for reads of unwritten LDS."""
    hipcc = _hipcc()
    out_lib = POISON_LIB if poison else LIB
    obj_dir = os.path.join(BUILD, "poison") if poison else BUILD
    if poison:
        extra_flags = (*extra_flags, "-DFA_POISON_LDS=1")
    os.makedirs(obj_dir, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(obj_dir, src.rsplit(".", 1)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmds.append([hipcc, *COMMON, *extra_flags, *lang, "-c",
                     os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = out_lib + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    # Loading resolves every symbol: a kernel whose host launch stub was not
    # emitted fails here, not at the first call.
    import ctypes
    ctypes.CDLL(tmp)
    os.replace(tmp, out_lib)
    if not poison:
        # The memory-side atomic throughput probe that bench.py runs.
        _run([hipcc, *[f for f in COMMON if f != "-fPIC"], "-x", "hip",
              os.path.join(CSRC, "atomic_probe.cpp"), "-o", PROBE], verbose)
    return out_lib


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
    print(build(verbose="--verbose" in sys.argv, poison=True))

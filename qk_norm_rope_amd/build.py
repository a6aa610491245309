"""Build the HIP libraries in-tree for gfx950: ``libqknr.so`` (the operation)
and ``libqknr_bench.so`` (the benchmark's streaming helpers).

    python -m qk_norm_rope_amd.build
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "qknr.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqknr.so")
BENCH_SRC = os.path.join(PKG, "csrc", "qknr_bench.hip")
BENCH_LIB = os.path.join(PKG, "libqknr_bench.so")
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled; ordinary float code is compiled to
# scalar v_fma/v_mul instead.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=" + ARCH,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libqknr.so)")


def _compile(src: str, lib: str, verbose: bool) -> str:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIP_FLAGS + ["-I" + INCLUDE, "-o", tmp, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 feature name and says so.
    noise = "not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if r.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    _compile(BENCH_SRC, BENCH_LIB, verbose)
    return _compile(SRC, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

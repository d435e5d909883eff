"""Builds libomerge.so in-tree with hipcc for gfx950.

    python -m ordered_merge_sorted_amd.build

The library lands in ordered_merge_sorted_amd/lib/, next to this package, so
that it travels with the source tree.  Packed FP32 instruction selection is
switched off (-packed-fp32-ops); the library has no floating point, so this
changes nothing in its code and only keeps every build of it uniform.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "libomerge.so")
SOURCES = [os.path.join(CSRC, "omerge.hip")]
INCLUDE = os.path.join(os.path.dirname(PKG), "include")

ARCH = "gfx950"
HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE,
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build_library(extra_flags=(), out: str = LIB, verbose: bool = False) -> str:
    """Compile the HIP sources into `out` (always recompiles)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s%s" % (r.returncode, r.stdout, r.stderr))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(sys.argv[1:], verbose=True))

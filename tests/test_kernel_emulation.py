"""CPU emulation of the HIP kernels against the oracle (no GPU).

The kernel headers are compiled unchanged as host C++ (tests/emu/) with
AddressSanitizer and UBSan, every lane a host thread, and run on seeded
cases: ragged sizes, every pointer phase, ring wraps, skew, empty sides,
unsorted input and nonsense partitions.  This checks the kernels' indexing
and barrier logic before they ever run on a GPU; the GPU tests then check
the compiled gfx950 code itself.
"""
import glob
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LLVM = "/opt/rocm/llvm"


def _asan_runtime():
    hits = glob.glob(os.path.join(LLVM, "lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[0] if hits else None


# Compile-time variants of the kernels: the default build (nontemporal
# streaming accesses) and plain accesses.
FLAG_SETS = {
    "default": [],
    "plain_access": ["-DOMERGE_NT_LOADS=0", "-DOMERGE_NT_STORES=0"],
}


@pytest.fixture(scope="module", params=sorted(FLAG_SETS))
def libemu(request, tmp_path_factory):
    clang = os.path.join(LLVM, "bin/clang++")
    rt = _asan_runtime()
    if not os.path.exists(clang) or rt is None:
        pytest.skip("host clang++ with the ASan runtime is not installed")
    out = str(tmp_path_factory.mktemp("emu") / ("libemu_%s.so" % request.param))
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared-libsan"]
    subprocess.check_call(
        [clang, "-std=c++20", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer", *san,
         *FLAG_SETS[request.param],
         "-I" + os.path.join(HERE, "emu"),
         "-I" + os.path.join(ROOT, "ordered_merge_sorted_amd", "csrc"),
         os.path.join(HERE, "emu", "emu.cpp"), "-o", out])
    return out, rt


CORE_GROUPS = ["small", "skew", "blocks", "direct", "production", "unsorted"]
# The typed, sort and batch groups exercise the same load and store helpers
# as the core groups, so they run in the default build only (keeps the CPU
# suite to a few minutes).
WIDE_GROUPS = ["orders", "sort", "batched", "batched_garbage"]


@pytest.mark.parametrize("group", CORE_GROUPS + WIDE_GROUPS)
def test_emulated_kernels_match_oracle(libemu, group):
    lib, rt = libemu
    if group in WIDE_GROUPS and not lib.endswith("libemu_default.so"):
        pytest.skip("typed, sort and batch groups run in the default build")
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, os.path.join(HERE, "emu", "run_emu_cases.py"), lib, group],
                       capture_output=True, text=True, timeout=1200, env=env)
    assert r.returncode == 0, (r.stdout[-4000:] + r.stderr[-6000:])
    assert "failures 0" in r.stdout

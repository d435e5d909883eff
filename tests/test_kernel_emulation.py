"""CPU emulation of the HIP kernels against the oracle (no GPU).

The kernel headers are compiled unchanged as host C++ (tests/emu/) with
AddressSanitizer and UBSan, every lane a host thread, and run on seeded
cases: ragged sizes, every pointer phase, ring wraps, skew, empty sides,
unsorted input, nonsense partitions and offsets, every key order, the sort
and the batched merge.  This checks the kernels' indexing and barrier logic
before they ever run on a GPU; the GPU tests then check the compiled gfx950
code itself.

Each (build, group) pair runs in a child process whose LD_PRELOAD holds the
sanitizer runtime.  The children spend most of their time in thread
barriers, so the module starts them all at once on a small pool and each
test waits for its own.
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

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
CORE_GROUPS = ["small", "skew", "blocks", "direct", "production", "unsorted", "search"]
# The typed, sort and batch groups, and the small shapes with each workgroup
# finding its own boundaries, exercise the same load and store helpers as
# the core groups, so they run in the default build only.
WIDE_GROUPS = ["orders", "sort", "batched", "batched_aligned", "batched_garbage", "multiway",
               "multiway_garbage", "small_self"]
JOBS = [(f, g) for f in sorted(FLAG_SETS) for g in CORE_GROUPS] + \
    [("default", g) for g in WIDE_GROUPS]
POOL = 6  # concurrent children (mostly waiting in barriers)


def _compile(flags_name, out_dir):
    clang = os.path.join(LLVM, "bin/clang++")
    out = os.path.join(out_dir, "libemu_%s.so" % flags_name)
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared-libsan"]
    subprocess.check_call(
        [clang, "-std=c++20", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer", *san,
         *FLAG_SETS[flags_name],
         "-I" + os.path.join(HERE, "emu"),
         "-I" + os.path.join(ROOT, "ordered_merge_sorted_amd", "csrc"),
         os.path.join(HERE, "emu", "emu.cpp"), "-o", out])
    return out


def _run(lib, rt, group):
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return subprocess.run([sys.executable, os.path.join(HERE, "emu", "run_emu_cases.py"), lib,
                           group], capture_output=True, text=True, timeout=1800, env=env)


@pytest.fixture(scope="module")
def emu_results(tmp_path_factory):
    """Compiles both builds, then starts every (build, group) run; returns
    {(build, group): future of the finished process}."""
    rt = _asan_runtime()
    if not os.path.exists(os.path.join(LLVM, "bin/clang++")) or rt is None:
        pytest.skip("host clang++ with the ASan runtime is not installed")
    out_dir = str(tmp_path_factory.mktemp("emu"))
    pool = ThreadPoolExecutor(POOL)
    libs = {f: pool.submit(_compile, f, out_dir) for f in FLAG_SETS}
    libs = {f: fut.result() for f, fut in libs.items()}
    # the longest runs first, so the pool's tail is short
    weight = {"batched": 6, "sort": 6, "small": 4, "small_self": 4, "direct": 3, "orders": 2}
    futures = {}
    for f, g in sorted(JOBS, key=lambda j: -weight.get(j[1], 1)):
        futures[(f, g)] = pool.submit(_run, libs[f], rt, g)
    yield futures
    pool.shutdown(wait=True)


@pytest.mark.parametrize("build,group", JOBS, ids=["%s-%s" % j for j in JOBS])
def test_emulated_kernels_match_oracle(emu_results, build, group):
    r = emu_results[(build, group)].result()
    assert r.returncode == 0, (r.stdout[-4000:] + r.stderr[-6000:])
    assert "failures 0" in r.stdout

"""bench.py's host-side helpers (no GPU): the flags it refuses, and the
check that ties the recorded HBM traffic to the kernel code it was measured
on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _hash_of(tmp_path, monkeypatch, texts):
    d = tmp_path / "ordered_merge_sorted_amd" / "csrc"
    d.mkdir(parents=True, exist_ok=True)
    for name, text in zip(bench.KERNEL_SOURCES, texts):
        (d / name).write_text(text)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return bench.kernel_source_hash()


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    code = ["int a = 1;\n", "int b = a + 2;  // two\n", "/* c */ int c = 3;\n"]
    base = _hash_of(tmp_path, monkeypatch, code)
    commented = ["// a new comment\nint a = 1;\n", "int b = a + 2;  // two, reworded\n",
                 "/* c,\n   over two lines */   int c = 3;\n"]
    assert _hash_of(tmp_path, monkeypatch, commented) == base
    changed = ["int a = 1;\n", "int b = a + 3;  // two\n", "/* c */ int c = 3;\n"]
    assert _hash_of(tmp_path, monkeypatch, changed) != base


def test_recorded_traffic_needs_the_matching_hash(tmp_path, monkeypatch):
    h = _hash_of(tmp_path, monkeypatch, ["int a;\n", "int b;\n", "int c;\n"])
    f = tmp_path / "traffic.md"
    monkeypatch.setattr(bench, "COUNTER_FILE", str(f))
    assert bench.recorded_traffic() is None  # no summary yet
    f.write_text("traffic_bytes_per_launch: 4.5e+09\nkernel_source_sha256_16: %s\n" % h)
    assert bench.recorded_traffic() == 4.5e9
    f.write_text("traffic_bytes_per_launch: 4.5e+09\nkernel_source_sha256_16: 0123456789abcdef\n")
    assert bench.recorded_traffic() is None  # taken on other code


@pytest.mark.parametrize("args", [["--gpus", "2"], ["--steps", "0"], ["--warmup", "-1"]])
def test_bench_refuses_bad_flags(args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert r.stdout.strip() == ""  # no JSON line

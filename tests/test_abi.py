"""The C ABI library on the CPU: it loads, exports every function that
include/omerge.h declares, and rejects bad arguments before touching a
device.  No call here launches work."""
import ctypes
import os
import re
import subprocess

import pytest

import ordered_merge_sorted_amd as om
from ordered_merge_sorted_amd import binding as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "omerge.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \t\*]*?\b([A-Za-z_]\w*)\s*\(", text, flags=re.M)
    return sorted(set(names) - {"defined"})


def test_header_declares_the_api():
    names = declared_functions()
    for want in ("merge_i32", "merge_kv", "omerge_co_rank", "omerge_partition",
                 "omerge_merge_segments_i32", "omerge_merge_segments_kv",
                 "omerge_status_string"):
        assert want in names, names


def test_library_exports_every_declared_symbol():
    lib = om.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", om.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = set(declared_functions()) - exported
    assert not missing, missing


def test_header_compiles_as_c():
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", HEADER],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_status_strings_and_version():
    lib = om.load_library()
    assert lib.omerge_status_string(0) == b"ok"
    assert lib.omerge_status_string(1) == b"invalid argument"
    assert lib.omerge_status_string(2) == b"size overflow"
    assert lib.omerge_status_string(3) == b"HIP error"
    assert lib.omerge_status_string(99) == b"unknown status"
    assert lib.omerge_version() >= 100
    assert lib.omerge_last_hip_error() == 0


def test_partition_count():
    assert om.partition_count(0, 4096) == 1
    assert om.partition_count(1, 4096) == 2
    assert om.partition_count(4096, 4096) == 2
    assert om.partition_count(4097, 4096) == 3
    assert om.partition_count(1 << 29, 87384) == 6145
    lib = om.load_library()
    assert lib.omerge_partition_count(100, 6) == -1       # not a multiple of 4
    assert lib.omerge_partition_count(100, 0) == -1
    assert lib.omerge_partition_count(-1, 4096) == -1
    assert lib.omerge_partition_count(100, (1 << 30) + 4) == -1


FAKE = 0x7F0000000000  # never dereferenced: every call below fails validation


def P(x):
    return ctypes.c_void_p(x)


@pytest.mark.parametrize("args,want", [
    ((P(0), 5, P(FAKE), 5, P(FAKE + 4096)), M.INVALID_ARG),          # A NULL, m > 0
    ((P(FAKE), 5, P(0), 5, P(FAKE + 4096)), M.INVALID_ARG),          # B NULL, n > 0
    ((P(FAKE), 5, P(FAKE + 64), 5, P(0)), M.INVALID_ARG),            # C NULL
    ((P(FAKE), -1, P(FAKE), 5, P(FAKE + 4096)), M.INVALID_ARG),      # negative m
    ((P(FAKE), 5, P(FAKE), -3, P(FAKE + 4096)), M.INVALID_ARG),      # negative n
    ((P(FAKE + 2), 5, P(FAKE + 64), 5, P(FAKE + 4096)), M.INVALID_ARG),  # misaligned A
    ((P(FAKE), 5, P(FAKE + 64), 5, P(FAKE + 4097)), M.INVALID_ARG),  # misaligned C
    ((P(FAKE), 5, P(FAKE + 64), 5, P(FAKE + 8)), M.INVALID_ARG),     # C overlaps A
    ((P(FAKE), 5, P(FAKE + 64), 5, P(FAKE + 40)), M.INVALID_ARG),    # C overlaps B
    ((P(FAKE), 1 << 62, P(FAKE), 1 << 62, P(FAKE)), M.OVERFLOW),     # m+n > 2^59
    ((P(0), 0, P(0), 0, P(0)), M.OK),                                # empty: no-op
])
def test_merge_i32_validation(args, want):
    lib = om.load_library()
    assert lib.merge_i32(*args, P(0)) == want


def test_merge_kv_validation():
    lib = om.load_library()
    f = lib.merge_kv
    a, av, b, bv = FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000
    ck, cv = FAKE + 0x4000, FAKE + 0x5000
    assert f(P(a), P(0), 4, P(b), P(bv), 4, P(ck), P(cv), P(0)) == M.INVALID_ARG
    assert f(P(a), P(av), 4, P(b), P(bv), 4, P(ck), P(ck + 8), P(0)) == M.INVALID_ARG  # outputs overlap
    assert f(P(a), P(av), 4, P(b), P(bv), 4, P(av), P(cv), P(0)) == M.INVALID_ARG      # C_keys over A_vals
    assert f(P(a), P(av), 4, P(b), P(bv), 4, P(ck), P(bv + 4), P(0)) == M.INVALID_ARG  # C_vals over B_vals
    assert f(P(0), P(0), 0, P(0), P(0), 0, P(0), P(0), P(0)) == M.OK


def test_typed_entry_validation():
    """Order codes outside the six kinds (optionally | 8) and payload widths
    other than 4 and 8 are rejected; the typed entries apply the same pointer,
    alignment and overlap checks as merge_i32 / merge_kv."""
    lib = om.load_library()
    a, av, b, bv = FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000
    ck, cv = FAKE + 0x4000, FAKE + 0x5000
    good = (0, 1, 2, 3, 4, 5, 8, 9, 10, 11, 12, 13)
    for bad in (6, 7, 14, 15, 16, -1, 1 << 20):
        assert lib.omerge_merge_keys(P(a), 4, P(b), 4, P(ck), bad, P(0)) == M.INVALID_ARG
        assert lib.omerge_merge_pairs(P(a), P(av), 4, P(b), P(bv), 4, P(ck), P(cv), bad, 4,
                                      P(0)) == M.INVALID_ARG
    for vb in (0, 2, 16, -4):
        assert lib.omerge_merge_pairs(P(a), P(av), 4, P(b), P(bv), 4, P(ck), P(cv), 0, vb,
                                      P(0)) == M.INVALID_ARG
    for order in good:
        wide = (order & 7) >= 3
        assert lib.omerge_merge_keys(P(a), 4, P(b), 4, P(a + 8), order, P(0)) == M.INVALID_ARG
        assert lib.omerge_merge_keys(P(0), 0, P(0), 0, P(0), order, P(0)) == M.OK
        # 64-bit keys must be 8-byte aligned; 32-bit keys need 4 bytes only
        rc = lib.omerge_merge_keys(P(a + 4), 0, P(b), 0, P(ck + 4), order, P(0))
        assert rc == M.OK  # empty: no pointer is used
        for vb in (4, 8):
            assert lib.omerge_merge_pairs(P(a), P(av), 4, P(b), P(bv), 4, P(ck), P(ck + 4),
                                          order, vb, P(0)) == M.INVALID_ARG
            assert lib.omerge_merge_pairs(P(0), P(0), 0, P(0), P(0), 0, P(0), P(0), order, vb,
                                          P(0)) == M.OK
            if vb == 8:  # misaligned 64-bit payload
                assert lib.omerge_merge_pairs(P(a), P(av + 4), 4, P(b), P(bv), 4, P(ck), P(cv),
                                              order, vb, P(0)) == M.INVALID_ARG
        if wide:  # misaligned 64-bit key
            assert lib.omerge_merge_keys(P(a + 4), 4, P(b), 4, P(ck), order, P(0)) == \
                M.INVALID_ARG
            # C of 8-byte keys reaching into A's bytes
            assert lib.omerge_merge_keys(P(a), 4, P(b), 4, P(a + 24), order, P(0)) == \
                M.INVALID_ARG
    assert (M.KEY_I32, M.KEY_U32, M.KEY_F32, M.KEY_I64, M.KEY_U64, M.KEY_F64,
            M.DESCENDING) == (0, 1, 2, 3, 4, 5, 8)
    text = open(HEADER).read()
    for i, name in enumerate(("I32", "U32", "F32", "I64", "U64", "F64")):
        assert re.search(r"\bOMERGE_KEY_%s = %d\b" % (name, i), text), name
    assert re.search(r"#define OMERGE_DESCENDING 8\b", text)


def test_batched_and_sort_validation():
    lib = om.load_library()
    a, av, b, bv = FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000
    ck, cv, ao, bo = FAKE + 0x4000, FAKE + 0x5000, FAKE + 0x6000, FAKE + 0x7000
    f = lib.omerge_merge_batched
    assert f(P(a), P(av), P(ao), 4, P(b), P(bv), P(bo), 4, 2, P(ck), P(cv), 0, 3, P(0)) == \
        M.INVALID_ARG                                                     # payload width
    assert f(P(a), P(0), P(ao), 4, P(b), P(0), P(bo), 4, 0, P(ck), P(0), 0, 0, P(0)) == \
        M.INVALID_ARG                                                     # no merges, data
    assert f(P(a), P(0), P(ao + 4), 4, P(b), P(0), P(bo), 4, 2, P(ck), P(0), 0, 0, P(0)) == \
        M.INVALID_ARG                                                     # offsets alignment
    assert f(P(a), P(0), P(0), 4, P(b), P(0), P(bo), 4, 2, P(ck), P(0), 0, 0, P(0)) == \
        M.INVALID_ARG                                                     # offsets NULL
    assert f(P(a), P(0), P(ck + 8), 4, P(b), P(0), P(bo), 4, 2, P(ck), P(0), 0, 0, P(0)) == \
        M.INVALID_ARG                                                     # C over offsets
    assert f(P(a), P(0), P(ao), 4, P(b), P(0), P(bo), 4, 2, P(a + 4), P(0), 0, 0, P(0)) == \
        M.INVALID_ARG                                                     # C over A
    assert f(P(a), P(0), P(ao), 4, P(b), P(0), P(bo), 4, 2, P(ck), P(0), 7, 0, P(0)) == \
        M.INVALID_ARG                                                     # order
    assert f(P(0), P(0), P(0), 0, P(0), P(0), P(0), 0, 0, P(0), P(0), 0, 0, P(0)) == M.OK
    assert f(P(0), P(0), P(0), 0, P(0), P(0), P(0), 0, 5, P(0), P(0), 0, 0, P(0)) == M.OK
    s = lib.omerge_sort
    assert s(P(a), P(0), P(ck), P(0), -1, 0, 0, P(0)) == M.INVALID_ARG  # negative n
    assert s(P(a), P(0), P(ck), P(0), 4, 6, 0, P(0)) == M.INVALID_ARG   # order
    assert s(P(a), P(av), P(ck), P(cv), 4, 0, 2, P(0)) == M.INVALID_ARG  # payload width
    assert s(P(a), P(0), P(a + 4), P(0), 4, 0, 0, P(0)) == M.INVALID_ARG  # partial overlap
    assert s(P(a), P(av), P(ck), P(ck + 8), 4, 0, 4, P(0)) == M.INVALID_ARG  # outputs overlap
    assert s(P(a), P(av), P(ck), P(a + 8), 4, 0, 4, P(0)) == M.INVALID_ARG  # vals out over keys in
    assert s(P(a + 4), P(0), P(ck), P(0), 4, 3, 0, P(0)) == M.INVALID_ARG  # 64-bit misaligned
    assert s(P(a), P(0), P(ck), P(0), 0, 0, 0, P(0)) == M.OK
    assert s(P(0), P(0), P(0), P(0), 0, 13, 8, P(0)) == M.OK
    r4 = lib.omerge_merge_runs4
    assert r4(P(a), P(ck), -1, 4, 0, P(0)) == M.INVALID_ARG      # negative n
    assert r4(P(a), P(ck), 4, 0, 0, P(0)) == M.INVALID_ARG       # run < 1
    assert r4(P(a), P(ck), 4, 4, 6, P(0)) == M.INVALID_ARG       # order
    assert r4(P(a), P(a + 4), 4, 4, 0, P(0)) == M.INVALID_ARG    # partial overlap
    assert r4(P(a), P(a), 4, 4, 0, P(0)) == M.INVALID_ARG        # in place
    assert r4(P(a + 4), P(ck), 4, 4, 3, P(0)) == M.INVALID_ARG   # 64-bit misaligned
    assert r4(P(0), P(ck), 4, 4, 0, P(0)) == M.INVALID_ARG       # NULL keys
    assert r4(P(a), P(ck), 0, 4, 0, P(0)) == M.OK
    assert r4(P(0), P(0), 0, 1, 13, P(0)) == M.OK


def test_order_code_of_dtypes():
    import torch
    assert om.order_code(torch.int32) == 0
    assert om.order_code(torch.float32, descending=True) == 10
    assert om.order_code(torch.int64) == 3
    assert om.order_code(torch.float64, descending=True) == 13
    if hasattr(torch, "uint32"):
        assert om.order_code(torch.uint32) == 1
    if hasattr(torch, "uint64"):
        assert om.order_code(torch.uint64, descending=True) == 12
    with pytest.raises(TypeError):
        om.order_code(torch.int16)


def test_stage_validation():
    lib = om.load_library()
    a, b, part, c = FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000
    assert lib.omerge_partition(P(a), 8, P(b), 8, 6, P(part), P(0)) == M.INVALID_ARG  # seg_len % 4
    assert lib.omerge_partition(P(a), 8, P(b), 8, 0, P(part), P(0)) == M.INVALID_ARG
    assert lib.omerge_partition(P(a), 8, P(b), 8, 8, P(0), P(0)) == M.INVALID_ARG
    assert lib.omerge_partition(P(a), 8, P(b), 8, 8, P(part + 4), P(0)) == M.INVALID_ARG
    assert lib.omerge_merge_segments_i32(P(a), 8, P(b), 8, P(0), 8, P(c), P(0)) == M.INVALID_ARG
    assert lib.omerge_merge_segments_i32(P(a), 8, P(b), 8, P(part), 10, P(c), P(0)) == M.INVALID_ARG
    assert lib.omerge_co_rank(P(a), 8, P(b), 8, P(0), 4, P(c), P(0)) == M.INVALID_ARG
    assert lib.omerge_co_rank(P(a), 8, P(b), 8, P(part), -1, P(c), P(0)) == M.INVALID_ARG
    assert lib.omerge_co_rank(P(a), 8, P(b), 8, P(0), 0, P(0), P(0)) == M.OK


def test_stage_outputs_must_not_overlap_inputs():
    """The stage calls reject an output that overlaps an input by address
    range: the partition array over A or B, a segment merge's output over
    its partition, and co-ranks over A, B or the queried ranks."""
    lib = om.load_library()
    a, b, part, c = FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000
    # 16 outputs in segments of 8: 3 partition entries (24 bytes)
    assert lib.omerge_partition(P(a), 8, P(b), 8, 8, P(a + 16), P(0)) == M.INVALID_ARG
    assert lib.omerge_partition(P(a), 8, P(b), 8, 8, P(b - 16), P(0)) == M.INVALID_ARG
    seg = lib.omerge_merge_segments_i32
    assert seg(P(a), 8, P(b), 8, P(c + 32), 8, P(c), P(0)) == M.INVALID_ARG    # part inside C
    assert seg(P(a), 8, P(b), 8, P(c - 16), 8, P(c), P(0)) == M.INVALID_ARG    # part runs into C
    kv = lib.omerge_merge_segments_kv
    av, bv, cv = FAKE + 0x4000, FAKE + 0x5000, FAKE + 0x6000
    assert kv(P(a), P(av), 8, P(b), P(bv), 8, P(part), 8, P(c), P(part + 8), P(0)) == \
        M.INVALID_ARG                                                          # C_vals over part
    assert kv(P(a), P(av), 8, P(b), P(bv), 8, P(cv + 8), 8, P(c), P(cv), P(0)) == M.INVALID_ARG
    cr = lib.omerge_co_rank
    k = FAKE + 0x7000
    assert cr(P(a), 8, P(b), 8, P(k), 4, P(a + 8), P(0)) == M.INVALID_ARG       # over A
    assert cr(P(a), 8, P(b), 8, P(k), 4, P(b + 24), P(0)) == M.INVALID_ARG      # over B
    assert cr(P(a), 8, P(b), 8, P(k), 4, P(k), P(0)) == M.INVALID_ARG           # in place
    assert cr(P(a), 8, P(b), 8, P(k), 4, P(k + 24), P(0)) == M.INVALID_ARG      # over k's tail
    cp = lib.omerge_stream_copy
    assert cp(P(a), 64, P(a + 128), P(0)) == M.INVALID_ARG   # overlap past the first 64 bytes
    assert cp(P(a), 64, P(a - 252), P(0)) == M.INVALID_ARG


def test_sizes_beyond_2p59_overflow():
    """Totals above 2^59 elements are refused before any byte size is formed
    (8-byte elements would otherwise overflow int64)."""
    lib = om.load_library()
    big = (1 << 59) + 1
    assert lib.merge_i32(P(FAKE), big, P(FAKE), 0, P(FAKE), P(0)) == M.OVERFLOW
    assert lib.merge_i32(P(FAKE), 1 << 58, P(FAKE), (1 << 58) + 1, P(FAKE), P(0)) == M.OVERFLOW
    assert lib.omerge_merge_keys(P(FAKE), big, P(FAKE), 0, P(FAKE), 3, P(0)) == M.OVERFLOW
    assert lib.omerge_sort(P(FAKE), P(0), P(FAKE), P(0), big, 3, 0, P(0)) == M.OVERFLOW
    assert lib.omerge_merge_runs4(P(FAKE), P(FAKE + 16), big, 4, 3, P(0)) == M.OVERFLOW
    assert lib.omerge_co_rank(P(FAKE), 4, P(FAKE), 4, P(FAKE), big, P(FAKE), P(0)) == M.OVERFLOW
    assert lib.omerge_stream_copy(P(FAKE), big, P(FAKE), P(0)) == M.OVERFLOW
    assert lib.omerge_partition_count(big, 4096) == -1
    assert lib.omerge_segment_length(big, 0, 0) == -1


def test_binding_rejects_bad_tensors():
    import torch
    cpu = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError):
        om.merge_i32(cpu, cpu)
    with pytest.raises(TypeError):
        om.merge_i32(cpu.float(), cpu)
    with pytest.raises(TypeError):
        om.merge_i32([1, 2], cpu)


def test_binding_stream_and_device_helpers():
    """An explicit stream is passed as its own handle; a device with no
    index (the current one) needs no device guard.  Neither touches a GPU."""
    import contextlib
    import torch

    class FakeStream:
        cuda_stream = 0x1234

    assert M._stream(torch.device("cuda", 0), FakeStream()) == 0x1234
    assert isinstance(M._on(torch.device("cuda")), contextlib.nullcontext)
    assert isinstance(M._on("cuda"), contextlib.nullcontext)
    cpu = torch.zeros(4, dtype=torch.int32)
    assert M._ptr(cpu[:0]) == 0 and M._ptr(cpu) == cpu.data_ptr()


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(M, "_lib", None)
    monkeypatch.setattr(M, "LIB", str(tmp_path / "absent.so"))
    with pytest.raises(M.OmergeError, match="not built"):
        M.load_library()


def test_no_alloc_rejects_totals_beyond_its_scratch():
    # Checked before anything is enqueued: the fake pointers are never used.
    lib = om.load_library()
    f = lib.merge_i32_no_alloc
    a, b, c = FAKE, FAKE + (1 << 34), FAKE + (1 << 36)
    assert f(P(a), (1 << 31), P(b), (1 << 31) + 4, P(c), P(0)) == M.SCRATCH_LIMIT
    assert f(P(a), (1 << 32) + 1, P(0), 0, P(c), P(0)) == M.SCRATCH_LIMIT
    assert lib.omerge_status_string(M.SCRATCH_LIMIT) == \
        b"exceeds the static scratch of merge_i32_no_alloc"
    # the usual argument checks come first
    assert f(P(0), 5, P(b), 5, P(c), P(0)) == M.INVALID_ARG
    assert f(P(a), 5, P(a + 8), 5, P(a + 16), P(0)) == M.INVALID_ARG
    assert f(P(0), 0, P(0), 0, P(0), P(0)) == M.OK

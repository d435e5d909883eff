"""HIP path against the CPU oracle, element by element (needs an MI355X).

Every output is compared exactly: a merge only permutes its input, so there
is no tolerance (page 'merge_path.cu' compares the same way).  Key-only
output cannot show the tie rule, so the co-ranks and the key+payload merge
are checked directly as well.
"""
import numpy as np
import pytest
import torch

import oracle
import ordered_merge_sorted_amd as om
from ordered_merge_sorted_amd.workloads import WORKLOADS, ORDER

pytestmark = pytest.mark.gpu

U31 = np.uint32(1 << 31)
DEV = torch.device("cuda:0")


def say(*a):
    print("[gpu-case]", *a, flush=True)


def dev(x, off=0):
    """numpy -> device tensor; with off > 0 the data starts `off` words into
    a larger allocation, so the pointer has a different 16-byte phase."""
    if x.dtype == np.uint32:
        x = x.view(np.int32)
    t = torch.from_numpy(np.ascontiguousarray(x))
    if off == 0:
        return t.to(DEV)
    big = torch.empty(x.size + off, dtype=t.dtype, device=DEV)
    big[off:] = t.to(DEV)
    return big[off:]


def host(t):
    return t.cpu().numpy()


def first_diff(got, want):
    bad = np.flatnonzero(got != want)
    return None if bad.size == 0 else (int(bad[0]), got[bad[0]], want[bad[0]], int(bad.size))


def assert_same(got, want, what):
    assert got.shape == want.shape, (what, got.shape, want.shape)
    d = first_diff(got, want)
    assert d is None, "%s: first difference at %d (got %r, want %r), %d differ" % ((what,) + d)


def pair(g, m, n, span):
    if span >= 1 << 32:
        lo, hi = -(1 << 31), 1 << 31
    else:
        lo = int(g.integers(-(1 << 31), (1 << 31) - span))
        hi = lo + span
    A = np.sort(g.integers(lo, hi, size=m, dtype=np.int64)).astype(np.int32)
    B = np.sort(g.integers(lo, hi, size=n, dtype=np.int64)).astype(np.int32)
    return A, B


def tags(m, n):
    return np.arange(m, dtype=np.uint32), (U31 + np.arange(n, dtype=np.uint32)).astype(np.uint32)


# --------------------------------------------------------------- small cases

@pytest.mark.parametrize("seed", range(12))
def test_random_i32_and_kv(seed):
    g = np.random.Generator(np.random.PCG64(1000 + seed))
    m, n = (int(x) for x in g.integers(0, 40000, size=2))
    span = int(g.choice([2, 16, 4096, 1 << 32]))
    A, B = pair(g, m, n, span)
    Av, Bv = tags(m, n)
    offs = [int(x) for x in g.integers(0, 4, size=6)] if seed % 2 else [0] * 6
    say("random", seed, m, n, span, offs)
    got = om.merge_i32(dev(A, offs[0]), dev(B, offs[1]))
    assert_same(host(got), oracle.merge_i32(A, B), "merge_i32")
    gk, gv = om.merge_kv(dev(A, offs[0]), dev(Av, offs[1]), dev(B, offs[2]), dev(Bv, offs[3]))
    wk, wv = oracle.merge_kv(A, Av, B, Bv)
    assert_same(host(gk), wk, "merge_kv keys")
    assert_same(host(gv).view(np.uint32), wv, "merge_kv payloads")


@pytest.mark.parametrize("seg_tiles", [1, 2, 3, 0])
def test_explicit_segments(seg_tiles):
    """Stage API with several segment lengths, including one that is not a
    whole number of tiles (short last tile in every segment)."""
    g = np.random.Generator(np.random.PCG64(77 + seg_tiles))
    m, n = 70001, 53333
    A, B = pair(g, m, n, 64)
    Av, Bv = tags(m, n)
    for kv, tile in ((False, 2048), (True, 2048)):  # the segment merge's tiles
        seg_len = tile * seg_tiles if seg_tiles else 4 * 1777
        say("segments", kv, seg_len)
        a, b = dev(A), dev(B)
        part = om.partition(a, b, seg_len)
        I = oracle.co_rank_all(A, B)
        ks = np.minimum(np.arange(part.numel()) * seg_len, m + n)
        assert_same(host(part), I[ks], "partition")
        if kv:
            gk, gv = om.merge_segments_kv(a, dev(Av), b, dev(Bv), part, seg_len)
            wk, wv = oracle.merge_kv(A, Av, B, Bv)
            assert_same(host(gk), wk, "keys")
            assert_same(host(gv).view(np.uint32), wv, "payloads")
        else:
            got = om.merge_segments_i32(a, b, part, seg_len)
            assert_same(host(got), oracle.merge_i32(A, B), "merge_segments_i32")


@pytest.mark.parametrize("seg_len,extra", [(4, 0), (4, 1), (12, 0), (12, 1)])
def test_partition_shape_switch(seg_len, extra):
    """The partition takes its 8-lane shape up to 49152 boundaries and its
    4-lane shape above; at exactly 49152 and 49153 boundaries (ragged last
    segment included) every co-rank and the segment merge stay exact."""
    total = seg_len * 49151 + extra  # 49152 boundaries, or one more for a 1-element tail
    g = np.random.Generator(np.random.PCG64(910 + seg_len + extra))
    m = total // 2 + 17
    A, B = pair(g, m, total - m, 300)
    a, b = dev(A), dev(B)
    say("partition switch", seg_len, total)
    part = om.partition(a, b, seg_len)
    assert part.numel() == 49152 + extra
    I = oracle.co_rank_all(A, B)
    ks = np.minimum(np.arange(part.numel()) * seg_len, total)
    assert_same(host(part), I[ks], "partition")
    got = om.merge_segments_i32(a, b, part, seg_len)
    assert_same(host(got), oracle.merge_i32(A, B), "merge_segments_i32")


def test_co_rank_every_k_with_ties():
    """Device co-rank at every output rank: here the A-first tie rule is
    visible even though the merged keys alone would not show it."""
    g = np.random.Generator(np.random.PCG64(5))
    for m, n, span in ((3000, 2000, 3), (1, 5000, 2), (4096, 4096, 1 << 32), (0, 77, 5), (77, 0, 5)):
        A, B = pair(g, m, n, span)
        say("co_rank", m, n, span)
        ks = torch.arange(m + n + 1, dtype=torch.int64, device=DEV)
        got = om.co_rank(dev(A), dev(B), ks)
        assert_same(host(got), oracle.co_rank_all(A, B), "co_rank")
    # out-of-range ranks are clamped into [0, m+n]
    A, B = pair(g, 10, 10, 4)
    got = om.co_rank(dev(A), dev(B), torch.tensor([-5, 0, 20, 99], dtype=torch.int64, device=DEV))
    assert list(host(got)) == [0, 0, 10, 10]


def test_worked_examples():
    import json, os
    gold = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    g1 = json.load(open(os.path.join(gold, "worked_example_corank.json")))
    A, B = np.array(g1["A"], np.int32), np.array(g1["B"], np.int32)
    ks = torch.tensor(g1["boundary_k"], dtype=torch.int64, device=DEV)
    assert list(host(om.co_rank(dev(A), dev(B), ks))) == g1["boundary_i"]
    C = host(om.merge_i32(dev(A), dev(B)))
    assert list(C[3:6]) == g1["thread1_output"]["values"]
    g2 = json.load(open(os.path.join(gold, "equal_element_case.json")))
    A, B = np.array(g2["A"], np.int32), np.array(g2["B"], np.int32)
    Av, Bv = tags(4, 4)
    gk, gv = om.merge_kv(dev(A), dev(Av), dev(B), dev(Bv))
    src = ["A%d" % v if v < U31 else "B%d" % (v - U31) for v in host(gv).view(np.uint32)]
    assert src == ["A0", "A1", "B0", "A2", "B1", "B2", "A3", "B3"]
    assert list(host(gk)) == [1, 1, 1, 2, 2, 2, 3, 4]


@pytest.mark.parametrize("layout", ["a_then_b", "b_then_a", "alternating", "equal_seams"])
def test_one_sided_tiles(layout):
    """Runs of one side longer than a tile (whole tiles from A alone or B
    alone), with mixed tiles at the seams."""
    if layout == "a_then_b":
        A, B = np.arange(0, 300000, dtype=np.int32), np.arange(300000, 500000, dtype=np.int32)
    elif layout == "b_then_a":
        A, B = np.arange(200000, 500000, dtype=np.int32), np.arange(0, 200000, dtype=np.int32)
    else:
        g = np.random.Generator(np.random.PCG64(99))
        runs = g.integers(1, 40000, size=24)
        A, B, v = [], [], 0
        for i, ln in enumerate(runs):
            (A if i % 2 == 0 else B).extend(range(v, v + int(ln)))
            v += int(ln) - (3 if layout == "equal_seams" else 0)
        A, B = np.sort(np.array(A, np.int32)), np.sort(np.array(B, np.int32))
    Av, Bv = tags(A.size, B.size)
    say("one-sided", layout, A.size, B.size)
    assert_same(host(om.merge_i32(dev(A), dev(B))), oracle.merge_i32(A, B), "i32")
    gk, gv = om.merge_kv(dev(A), dev(Av), dev(B), dev(Bv))
    wk, wv = oracle.merge_kv(A, Av, B, Bv)
    assert_same(host(gk), wk, "kv keys")
    assert_same(host(gv).view(np.uint32), wv, "kv payloads")


@pytest.mark.parametrize("two_searches", [False, True])
def test_direct_global_memory_kernels(two_searches):
    """The no-LDS ablation kernels give the same output at every slice size."""
    g = np.random.Generator(np.random.PCG64(321))
    for m, n, span in ((40000, 30001, 64), (0, 5000, 8), (7777, 1, 1 << 32)):
        A, B = pair(g, m, n, span)
        want = oracle.merge_i32(A, B)
        for per in (1, 4, 16, 64, 256):
            say("direct", two_searches, m, n, per)
            got = om.merge_i32_direct(dev(A), dev(B), per_thread=per, two_searches=two_searches)
            assert_same(host(got), want, "direct per=%d" % per)


EDGE = [
    (0, 0), (1, 0), (0, 1), (1, 1), (3, 0), (0, 4095), (4095, 1), (4096, 0), (4097, 0),
    (2048, 2048), (2049, 2048), (1, 100000), (100000, 1), (12289, 4093),
]


@pytest.mark.parametrize("m,n", EDGE)
def test_edge_sizes(m, n):
    g = np.random.Generator(np.random.PCG64(m * 7919 + n))
    A, B = pair(g, m, n, 8)
    Av, Bv = tags(m, n)
    say("edge", m, n)
    assert_same(host(om.merge_i32(dev(A), dev(B))), oracle.merge_i32(A, B), "i32")
    gk, gv = om.merge_kv(dev(A), dev(Av), dev(B), dev(Bv))
    wk, wv = oracle.merge_kv(A, Av, B, Bv)
    assert_same(host(gk), wk, "kv keys")
    assert_same(host(gv).view(np.uint32), wv, "kv payloads")


def test_int32_extremes_and_all_equal():
    imin, imax = -(1 << 31), (1 << 31) - 1
    cases = [
        (np.array([imin, imin, -1, 0, imax, imax], np.int32), np.array([imin, 0, 0, imax], np.int32)),
        (np.full(10000, 7, np.int32), np.full(9000, 7, np.int32)),
        (np.full(5000, imax, np.int32), np.full(5000, imin, np.int32)),
        (np.full(5000, imin, np.int32), np.full(5000, imax, np.int32)),
    ]
    for A, B in cases:
        Av, Bv = tags(A.size, B.size)
        say("extremes", A.size, B.size)
        assert_same(host(om.merge_i32(dev(A), dev(B))), oracle.merge_i32(A, B), "i32")
        gk, gv = om.merge_kv(dev(A), dev(Av), dev(B), dev(Bv))
        wk, wv = oracle.merge_kv(A, Av, B, Bv)
        assert_same(host(gv).view(np.uint32), wv, "kv payloads")


def test_uint32_payload_dtype():
    if not hasattr(torch, "uint32"):
        pytest.skip("torch has no uint32")
    A, B = pair(np.random.Generator(np.random.PCG64(3)), 3000, 2000, 10)
    Av, Bv = tags(3000, 2000)
    av = torch.from_numpy(Av).to(DEV)
    bv = torch.from_numpy(Bv).to(DEV)
    gk, gv = om.merge_kv(dev(A), av, dev(B), bv)
    assert gv.dtype == torch.uint32
    assert_same(gv.cpu().numpy(), oracle.merge_kv(A, Av, B, Bv)[1], "uint32 payloads")


def test_non_default_stream():
    g = np.random.Generator(np.random.PCG64(9))
    A, B = pair(g, 300000, 200000, 1000)
    a, b = dev(A), dev(B)
    torch.cuda.synchronize()
    s = torch.cuda.Stream(DEV)
    with torch.cuda.stream(s):
        out = torch.empty(A.size + B.size, dtype=torch.int32, device=DEV)
        om.merge_i32(a, b, out=out)
        ev = torch.cuda.Event()
        ev.record(s)
    ev.synchronize()
    assert_same(host(out), oracle.merge_i32(A, B), "stream")


def test_calls_on_two_streams_at_once():
    """Sorts, a key+payload merge and a batched merge in flight together on
    two streams: each call takes its temporaries on its own stream and the
    library keeps no state between calls, so every result matches the
    oracle as it does alone."""
    g = np.random.Generator(np.random.PCG64(12))
    K1 = g.integers(-(1 << 31), 1 << 31, size=3_000_017, dtype=np.int64).astype(np.int32)
    K2 = g.integers(-50, 50, size=2_100_001, dtype=np.int64).astype(np.int32)
    A, B = pair(g, 1_500_000, 1_200_001, 5000)
    Av, Bv = tags(A.size, B.size)
    P, L = 700, 1000
    X = np.sort(g.integers(0, 1 << 20, size=(P, L)), axis=1).astype(np.int32).reshape(-1)
    Y = np.sort(g.integers(0, 1 << 20, size=(P, L)), axis=1).astype(np.int32).reshape(-1)
    offs = np.arange(0, P * L + 1, L, dtype=np.int64)
    k1, k2, a, av, b, bv = dev(K1), dev(K2), dev(A), dev(Av), dev(B), dev(Bv)
    x, y, o = dev(X), dev(Y), torch.from_numpy(offs).to(DEV)
    torch.cuda.synchronize()
    say("two streams")
    s1, s2 = torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)
    with torch.cuda.stream(s1):
        got1 = om.sort(k1)
        gotb = om.merge_batched(x, o, y, o)
    with torch.cuda.stream(s2):
        gk, gv = om.merge_kv(a, av, b, bv)
        got2 = om.sort(k2)
    torch.cuda.synchronize()
    assert_same(host(got1), oracle.sort(K1), "sort on stream 1")
    assert_same(host(gotb), oracle.merge_batched(X, offs, Y, offs), "batched on stream 1")
    wk, wv = oracle.merge_kv(A, Av, B, Bv)
    assert_same(host(gk), wk, "merge_kv keys on stream 2")
    assert_same(host(gv).view(np.uint32), wv, "merge_kv payloads on stream 2")
    assert_same(host(got2), oracle.sort(K2), "sort on stream 2")


def test_graph_capture_and_replay():
    """The merge paths that allocate nothing (merge_i32_no_alloc, and the
    two stages with a preallocated partition and output) captured once in a
    HIP graph, then replayed on new data written into the same inputs, with
    eager work and synchronisations between replays: every replay matches
    the oracle on its data."""
    g = np.random.Generator(np.random.PCG64(13))
    m, n = 1_000_003, 777_777
    a = torch.empty(m, dtype=torch.int32, device=DEV)
    b = torch.empty(n, dtype=torch.int32, device=DEV)
    out1 = torch.empty(m + n, dtype=torch.int32, device=DEV)
    out2 = torch.empty(m + n, dtype=torch.int32, device=DEV)
    seg_len = om.segment_length(m, n)
    part = torch.empty(om.partition_count(m + n, seg_len), dtype=torch.int64, device=DEV)

    def load(span):
        A, B = pair(g, m, n, span)
        a.copy_(torch.from_numpy(A))
        b.copy_(torch.from_numpy(B))
        return A, B

    load(1000)
    om.merge_i32_no_alloc(a, b, out1)  # the first call on a device looks up its scratch
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        om.merge_i32_no_alloc(a, b, out1)
        om.partition(a, b, seg_len, out=part)
        om.merge_segments_i32(a, b, part, seg_len, out=out2)
    for r, span in enumerate((1 << 32, 7, 100000, 1 << 32)):
        A, B = load(span)
        out1.fill_(-1)
        out2.fill_(-1)
        torch.cuda.synchronize()
        say("graph replay", r, span)
        graph.replay()
        torch.cuda.synchronize()
        want = oracle.merge_i32(A, B)
        assert_same(host(out1), want, "replay %d, merge_i32_no_alloc" % r)
        assert_same(host(out2), want, "replay %d, partition + merge_segments_i32" % r)
        _check_partition(A, B, host(part), seg_len)


def test_repeatable_and_preallocated_out():
    g = np.random.Generator(np.random.PCG64(10))
    A, B = pair(g, 123457, 98765, 50)
    a, b = dev(A), dev(B)
    out = torch.full((A.size + B.size,), -1, dtype=torch.int32, device=DEV)
    first = host(om.merge_i32(a, b, out=out)).copy()
    for _ in range(3):
        assert_same(host(om.merge_i32(a, b, out=out)), first, "repeat")
    assert_same(first, oracle.merge_i32(A, B), "oracle")


@pytest.mark.parametrize("off", [1, 2, 3])
def test_unaligned_outputs(off):
    """Outputs that start `off` words past a 16-byte boundary: the 4-byte-key
    merges then store tiles word by word instead of as 16-byte vectors.
    Several segments and a ragged tail; every output against the oracle and
    the words around each output untouched."""
    g = np.random.Generator(np.random.PCG64(40 + off))
    A, B = pair(g, 21011 + off, 17003, 300)
    Av, Bv = tags(A.size, B.size)
    t = A.size + B.size
    say("unaligned outputs", off, A.size, B.size)
    sentinel = -123456789

    def window(o):
        buf = torch.full((t + 8,), sentinel, dtype=torch.int32, device=DEV)
        return buf, buf[o:o + t]

    buf, out = window(off)
    om.merge_i32(dev(A), dev(B), out=out)
    bk, ok_ = window(off)
    bv, ov = window((off + 1) % 4)
    om.merge_kv(dev(A), dev(Av), dev(B), dev(Bv), out_keys=ok_, out_vals=ov)
    wk, wv = oracle.merge_kv(A, Av, B, Bv)
    assert_same(host(out), oracle.merge_i32(A, B), "merge_i32, unaligned output")
    assert_same(host(ok_), wk, "merge_kv keys, unaligned output")
    assert_same(host(ov).view(np.uint32), wv, "merge_kv payloads, unaligned output")
    for b, o in ((buf, off), (bk, off), (bv, (off + 1) % 4)):
        h = host(b)
        assert np.all(h[:o] == sentinel) and np.all(h[o + t:] == sentinel), "write outside output"


@pytest.mark.parametrize("off", [0, 1])
def test_unaligned_outputs_wide(off):
    """int64 and float64 keys into outputs `off` elements (8 bytes) past a
    16-byte boundary: aligned outputs take the register-store merge (quad
    transpose), unaligned ones the staged one.  Several segments and a
    ragged tail; every output against the oracle, guard words untouched."""
    g = np.random.Generator(np.random.PCG64(50 + off))
    for dtype in (np.int64, np.float64):
        A, B = typed_pair(g, dtype, False, 30011 + off, 25013)
        t = A.size + B.size
        say("unaligned wide outputs", np.dtype(dtype).name, off, A.size, B.size)
        buf = torch.full((t + 4,), -7, dtype=torch.int64, device=DEV)
        out = buf[off:off + t]
        if dtype == np.float64:
            out = out.view(torch.float64)
        om.merge(dev_typed(A), dev_typed(B), out=out)
        assert_same(host_bits(out), as_bits(oracle.merge_keys(A, B, False)), "wide, offset output")
        h = host(buf)
        assert np.all(h[:off] == -7) and np.all(h[off + t:] == -7), "write outside output"


def test_unsorted_input_returns():
    """Sortedness is not checked; unsorted input must still return (the
    kernels' loops are bounded) with an output of the right size."""
    g = np.random.Generator(np.random.PCG64(11))
    A = g.integers(-100, 100, size=50000).astype(np.int32)
    B = g.integers(-100, 100, size=30000).astype(np.int32)
    out = om.merge_i32(dev(A), dev(B))
    torch.cuda.synchronize()
    assert out.numel() == 80000


# ------------------------------------------------------ key types and orders

KEY_DTYPES = [np.int32, np.uint32, np.float32, np.int64, np.uint64, np.float64]
TYPED = [(d, r) for d in KEY_DTYPES for r in (False, True)]
TYPED_IDS = ["%s-%s" % (np.dtype(d).name, "desc" if r else "asc") for d, r in TYPED]
_TORCH = {np.dtype(np.int32): torch.int32, np.dtype(np.uint32): getattr(torch, "uint32", None),
          np.dtype(np.float32): torch.float32, np.dtype(np.int64): torch.int64,
          np.dtype(np.uint64): getattr(torch, "uint64", None),
          np.dtype(np.float64): torch.float64}


def dev_typed(x, off=0):
    """Keys or payloads of any 4- or 8-byte dtype to a device tensor of the
    matching torch dtype (moved as signed-integer bits of the same width)."""
    x = np.ascontiguousarray(x)
    tdt = _TORCH[x.dtype]
    bits = np.int32 if x.dtype.itemsize == 4 else np.int64
    t = torch.from_numpy(x.view(bits))
    if off:
        big = torch.empty(x.size + off, dtype=t.dtype, device=DEV)
        big[off:] = t.to(DEV)
        t = big[off:]
    else:
        t = t.to(DEV)
    return t.view(tdt)


def host_bits(t):
    bits = torch.int32 if t.element_size() == 4 else torch.int64
    ubits = np.uint32 if t.element_size() == 4 else np.uint64
    return t.view(bits).cpu().numpy().view(ubits)


def as_bits(x):
    return np.ascontiguousarray(x).view(np.uint32 if x.dtype.itemsize == 4 else np.uint64)


_FLOAT_POOLS = {}


def float_pool(dtype):
    """About 2000 distinct values of a float dtype, signed zeros, infinities,
    subnormals and NaNs of both signs among them, sorted with the oracle's
    totalOrder relation."""
    if dtype not in _FLOAT_POOLS:
        import functools
        g = np.random.Generator(np.random.PCG64(77))
        if dtype == np.float32:
            special = np.array([0xFFC00000, 0xFFFFFFFF, 0xFF800001, 0xFF800000, 0xFF7FFFFF,
                                0x80800000, 0x80000001, 0x80000000, 0x00000000, 0x00000001,
                                0x00800000, 0x7F7FFFFF, 0x7F800000, 0x7F800001, 0x7FC00000,
                                0x7FFFFFFF], dtype=np.uint32)
            anybits = g.integers(0, 1 << 32, size=500, dtype=np.uint64).astype(np.uint32)
        else:
            special = np.array([0xFFF8000000000000, 0xFFFFFFFFFFFFFFFF, 0xFFF0000000000001,
                                0xFFF0000000000000, 0xFFEFFFFFFFFFFFFF, 0x8010000000000000,
                                0x8000000000000001, 0x8000000000000000, 0x0000000000000000,
                                0x0000000000000001, 0x0010000000000000, 0x7FEFFFFFFFFFFFFF,
                                0x7FF0000000000000, 0x7FF0000000000001, 0x7FF8000000000000,
                                0x7FFFFFFFFFFFFFFF], dtype=np.uint64)
            anybits = g.integers(0, 1 << 64, size=500, dtype=np.uint64)
        ubits = special.dtype.type
        finite = (g.standard_normal(1500) * 1e3).astype(dtype).view(ubits)
        vals = np.unique(np.concatenate([special, finite, anybits.astype(ubits)])).view(dtype)

        def cmp(x, y):
            if not oracle.key_le(dtype, x, y):
                return 1
            return 0 if oracle.key_le(dtype, y, x) else -1
        _FLOAT_POOLS[dtype] = np.array(sorted(vals.tolist(), key=functools.cmp_to_key(
            lambda a, b: cmp(dtype(a), dtype(b)))), dtype=dtype)
    return _FLOAT_POOLS[dtype]


def typed_pair(g, dtype, desc, m, n):
    if dtype in (np.float32, np.float64):
        pool = float_pool(dtype)
        A = pool[np.sort(g.integers(0, pool.size, size=m))]
        B = pool[np.sort(g.integers(0, pool.size, size=n))]
    else:
        info = np.iinfo(dtype)
        span = int(g.choice([3, 5000, 0]))
        if span == 0:  # the whole range of the type
            A = np.sort(g.integers(info.min, info.max, size=m, dtype=dtype, endpoint=True))
            B = np.sort(g.integers(info.min, info.max, size=n, dtype=dtype, endpoint=True))
        else:
            lo = int(g.integers(info.min, int(info.max) - span, dtype=dtype))
            A = np.sort(g.integers(lo, lo + span, size=m, dtype=dtype))
            B = np.sort(g.integers(lo, lo + span, size=n, dtype=dtype))
    if desc:
        A, B = A[::-1], B[::-1]
    return np.ascontiguousarray(A), np.ascontiguousarray(B)


def tags64(m, n):
    return (np.arange(m, dtype=np.uint64),
            (np.uint64(1 << 63) + np.arange(n, dtype=np.uint64)).astype(np.uint64))


def needs_torch_dtype(dtype):
    if _TORCH[np.dtype(dtype)] is None:
        pytest.skip("this torch has no %s dtype" % np.dtype(dtype).name)


@pytest.mark.parametrize("dtype,desc", TYPED, ids=TYPED_IDS)
def test_typed_keys_and_pairs(dtype, desc):
    """Every key type and direction, keys only and with 4- and 8-byte
    payloads, several tiles plus a ragged tail, several pointer phases;
    output bits against the oracle."""
    needs_torch_dtype(dtype)
    g = np.random.Generator(np.random.PCG64(500 + TYPED.index((dtype, desc))))
    wide = np.dtype(dtype).itemsize == 8
    for c in range(4):
        m, n = (int(x) for x in g.integers(0, 60000, size=2))
        if c == 3:
            m = 0
        A, B = typed_pair(g, dtype, desc, m, n)
        # offsets in elements: 64-bit arrays keep their 8-byte alignment
        offs = [int(x) for x in g.integers(0, 4, size=6)]
        say("typed", np.dtype(dtype).name, desc, m, n, offs)
        got = om.merge(dev_typed(A, offs[0]), dev_typed(B, offs[1]), descending=desc)
        assert got.dtype == _TORCH[np.dtype(dtype)]
        want = oracle.merge_keys(A, B, desc)
        assert_same(host_bits(got), as_bits(want), "typed keys")
        for tagger in (tags, tags64):
            Av, Bv = tagger(m, n)
            if tagger is tags64 and _TORCH[np.dtype(np.uint64)] is None:
                Av, Bv = Av.view(np.int64), Bv.view(np.int64)
            gk, gv = om.merge_pairs(dev_typed(A, offs[2]), dev_typed(Av, offs[3]),
                                    dev_typed(B, offs[4]), dev_typed(Bv, offs[5]),
                                    descending=desc)
            wk, wv = oracle.merge_pairs(A, Av, B, Bv, desc)
            what = "typed pair (%d-byte payloads)" % Av.dtype.itemsize
            assert_same(host_bits(gk), as_bits(wk), what + " keys")
            assert_same(host_bits(gv), as_bits(wv), what + " payloads")
        if wide and dtype != np.float64:
            # one shared high word: keys differ in the low 32 bits only
            hi = -(5 << 32) if (dtype == np.int64 and c % 2) else (3 << 32)
            vals = (np.int64(hi) + g.integers(0, 1 << 32, size=4000)).astype(dtype)
            A2, B2 = np.sort(g.choice(vals, 2500)), np.sort(g.choice(vals, 1500))
            if desc:
                A2, B2 = A2[::-1].copy(), B2[::-1].copy()
            got = om.merge(dev_typed(A2), dev_typed(B2), descending=desc)
            assert_same(host_bits(got), as_bits(oracle.merge_keys(A2, B2, desc)),
                        "low-word keys")


def test_i32_order_code_is_merge_i32():
    g = np.random.Generator(np.random.PCG64(611))
    A, B = pair(g, 30000, 20000, 64)
    assert_same(host(om.merge(dev(A), dev(B))), host(om.merge_i32(dev(A), dev(B))), "i32 order 0")


@pytest.mark.parametrize("dtype,desc", [(np.float32, True), (np.uint32, False),
                                        (np.int64, False), (np.float64, True)],
                         ids=["float32-desc", "uint32-asc", "int64-asc", "float64-desc"])
def test_typed_large(dtype, desc):
    """2^24 + 2^24 keys, and pairs with 4- and 8-byte payloads, of orders
    other than int32 ascending (thousands of tiles)."""
    needs_torch_dtype(dtype)
    g = np.random.Generator(np.random.PCG64(613))
    m = n = 1 << 24
    A, B = typed_pair(g, dtype, desc, m, n)
    say("typed large", np.dtype(dtype).name, desc)
    got = om.merge(dev_typed(A), dev_typed(B), descending=desc)
    assert_same(host_bits(got), as_bits(oracle.merge_keys(A, B, desc)), "typed large")
    del got
    for tagger in (tags, tags64):
        Av, Bv = tagger(m, n)
        if tagger is tags64 and _TORCH[np.dtype(np.uint64)] is None:
            Av, Bv = Av.view(np.int64), Bv.view(np.int64)
        gk, gv = om.merge_pairs(dev_typed(A), dev_typed(Av), dev_typed(B), dev_typed(Bv),
                                descending=desc)
        wk, wv = oracle.merge_pairs(A, Av, B, Bv, desc)
        assert_same(host_bits(gk), as_bits(wk), "typed large pair keys")
        assert_same(host_bits(gv), as_bits(wv), "typed large pair payloads")
        del gk, gv


# ------------------------------------------------- batched merges and the sort


def unsorted_typed(g, dtype, n):
    """Unsorted keys: floats from the totalOrder pool (specials included),
    integers with many ties or over the whole range."""
    if dtype in (np.float32, np.float64):
        pool = float_pool(dtype)
        return pool[g.integers(0, pool.size, size=n)]
    info = np.iinfo(dtype)
    if g.random() < 0.5:
        return g.integers(0, 40, size=n).astype(dtype)
    return g.integers(info.min, info.max, size=n, dtype=dtype, endpoint=True)


@pytest.mark.parametrize("dtype,desc", TYPED, ids=TYPED_IDS)
def test_sort_keys_and_pairs(dtype, desc):
    """Stable merge sort of every key type and order, keys only and with
    4- and 8-byte payloads, around the block sort's run lengths (2,048,
    4,096, 8,192 and 16,384 elements, by shape) and over many passes; output
    bits against the oracle's stable sort."""
    needs_torch_dtype(dtype)
    g = np.random.Generator(np.random.PCG64(700 + TYPED.index((dtype, desc))))
    for n in (0, 1, 1023, 1024, 2047, 2048, 2049, 4095, 4097, 8191, 8192, 8193, 16383, 16384,
              16385, 32769, 70001, int(g.integers(100000, 300000))):
        K = np.ascontiguousarray(unsorted_typed(g, dtype, n))
        say("sort", np.dtype(dtype).name, desc, n)
        got = om.sort(dev_typed(K), descending=desc)
        assert_same(host_bits(got), as_bits(oracle.sort(K, descending=desc)), "sorted keys")
        for vdt in (np.uint32, np.int64):
            V = (np.arange(n) * 7 + 3).astype(vdt)
            gk, gv = om.sort(dev_typed(K), dev_typed(V), descending=desc)
            wk, wv = oracle.sort(K, V, descending=desc)
            assert_same(host_bits(gk), as_bits(wk), "sorted pair keys")
            assert_same(host_bits(gv), as_bits(wv), "sorted pair payloads")


@pytest.mark.parametrize("off", [0, 1, 2])
def test_sort_unaligned_outputs(off):
    """Sorts of int32 keys (alone and with int32 payloads) into outputs `off`
    words past a 16-byte boundary: aligned outputs take the passes that
    store from registers, unaligned ones the staged passes.  Many passes and
    a ragged last pair; every output against the oracle and the words
    around each output untouched."""
    g = np.random.Generator(np.random.PCG64(760 + off))
    n = 300007
    K = g.integers(-1000, 1000, size=n).astype(np.int32)
    V = np.arange(n, dtype=np.int32)
    say("sort unaligned outputs", off, n)
    sentinel = -987654321

    def window(o):
        buf = torch.full((n + 8,), sentinel, dtype=torch.int32, device=DEV)
        return buf, buf[o:o + n]

    bk, ok_ = window(off)
    om.sort(dev(K), out=ok_)
    pk, pko = window(off)
    pv, pvo = window((off + 2) % 4)
    om.sort(dev(K), dev(V), out=pko, out_vals=pvo)
    assert_same(host(ok_), oracle.sort(K), "sorted keys, offset output")
    wk, wv = oracle.sort(K, V)
    assert_same(host(pko), wk, "sorted pair keys, offset output")
    assert_same(host(pvo), wv, "sorted pair payloads, offset output")
    for b, o in ((bk, off), (pk, off), (pv, (off + 2) % 4)):
        h = host(b)
        assert np.all(h[:o] == sentinel) and np.all(h[o + n:] == sentinel), "write outside output"


def test_sort_in_place_and_large():
    """In-place sort (out = input), and 2^24 int32 keys with payloads (11
    merge passes after the block sort's 8,192-pair runs)."""
    g = np.random.Generator(np.random.PCG64(733))
    K = g.integers(-(1 << 31), 1 << 31, size=300000, dtype=np.int64).astype(np.int32)
    t = dev(K)
    om.sort(t, out=t)
    assert_same(host(t), oracle.sort(K), "in place")
    n = 1 << 24
    K = g.integers(0, 1 << 20, size=n).astype(np.int32)
    V = np.arange(n, dtype=np.uint32)
    say("sort large", n)
    gk, gv = om.sort(dev(K), dev(V))
    wk, wv = oracle.sort(K, V)
    assert_same(host(gk), wk, "large sort keys")
    assert_same(host(gv).view(np.uint32), wv, "large sort payloads")


@pytest.mark.parametrize("dtype,desc", [(np.int32, False), (np.float32, True), (np.int64, True),
                                        (np.float64, False)],
                         ids=["int32", "float32-desc", "int64-desc", "float64"])
def test_sort_keys_many_passes(dtype, desc):
    """Key-only sorts past the block sort's runs: sizes that leave the last
    pair of runs short or missing, an even and an odd number of passes, keys
    over the whole range and keys with four values only.  Output bits
    against the oracle's stable sort."""
    needs_torch_dtype(dtype)
    g = np.random.Generator(np.random.PCG64(780 + np.dtype(dtype).itemsize + 2 * desc))
    tile = 16384  # the block sort's runs of 4- and 8-byte keys alone
    for n in (4 * tile, 4 * tile + 1, 5 * tile - 3, 7 * tile + 11, 16 * tile,
              16 * tile + 3 * tile + 5, 64 * tile + 2 * 16 * tile + 999, (1 << 22) + 77777):
        for few in (False, True):
            if few:
                K = np.array([-7, 0, 3, 12], dtype=dtype)[g.integers(0, 4, size=n)]
            else:
                K = np.ascontiguousarray(unsorted_typed(g, dtype, n))
            say("sort many passes", np.dtype(dtype).name, desc, n, few)
            got = om.sort(dev_typed(K), descending=desc)
            assert_same(host_bits(got), as_bits(oracle.sort(K, descending=desc)),
                        "sorted keys (n=%d, few=%s)" % (n, few))


def test_sort_headline_size():
    """2^28 int32 keys iid uniform over the int32 range (the size the sort
    is timed at).  Keys alone have one sorted order, so the output is
    compared bit for bit with numpy's sort of the input (the oracle's merge
    sort takes minutes at this size)."""
    n = 1 << 28
    g = np.random.Generator(np.random.PCG64(791))
    K = g.integers(-(1 << 31), 1 << 31, size=n, dtype=np.int64).astype(np.int32)
    say("sort headline size", n)
    got = om.sort(dev(K))
    want = np.sort(K)
    h = host(got)
    assert np.array_equal(h, want), "2^28 sort differs from the sorted input"
    del got
    torch.cuda.empty_cache()


def test_stream_copy_reference():
    """The bandwidth reference copy (omerge_stream_copy): every size class
    (empty, a few words, one 64-lane workgroup and its neighbours, a ragged
    large size) and every source and destination word phase, so both the
    16-byte path (same phase) and the word path (different phases) run;
    the copy must equal the source and leave the words around it alone."""
    g = np.random.Generator(np.random.PCG64(830))
    sentinel = -55555
    for n in (0, 1, 3, 5, 255, 256, 257, 1000003, (1 << 20) + 7):
        src_h = g.integers(-(1 << 31), 1 << 31, size=n + 8, dtype=np.int64).astype(np.int32)
        src_d = dev(src_h)
        for so in range(4):
            for do in range(4):
                buf = torch.full((n + 16,), sentinel, dtype=torch.int32, device=DEV)
                out = buf[4 + do:4 + do + n]
                om.stream_copy(src_d[so:so + n], out=out)
                h = host(buf)
                assert np.array_equal(h[4 + do:4 + do + n], src_h[so:so + n]), (n, so, do)
                assert np.all(h[:4 + do] == sentinel) and np.all(h[4 + do + n:] == sentinel), \
                    (n, so, do)


def sorted_runs(g, dtype, desc, n, run, few):
    """n keys whose runs of `run` are each sorted in the key order (the
    oracle's stable sort per run)."""
    if few:
        K = np.array([0, 3, 12, 40], dtype=dtype)[g.integers(0, 4, size=n)]
    else:
        K = np.ascontiguousarray(unsorted_typed(g, dtype, n))
    for s0 in range(0, n, run):
        K[s0:s0 + run] = oracle.sort(K[s0:s0 + run], descending=desc)
    return K


@pytest.mark.parametrize("dtype,desc", TYPED, ids=TYPED_IDS)
def test_merge_runs4_against_oracle(dtype, desc):
    """One 4-way merge pass (omerge_merge_runs4) of every key type and order
    against the oracle's k-way pass: runs shorter than, equal to and longer
    than a cell's bound (4,096 keys per pair for 4-byte keys, 2,048 for
    8-byte), groups of one to four runs at the end, a short last run, keys
    over the whole range and keys with four values (ties across all four
    runs and across sample points), and a run of the whole input (a copy)."""
    needs_torch_dtype(dtype)
    g = np.random.Generator(np.random.PCG64(800 + TYPED.index((dtype, desc))))
    q = 4096 if np.dtype(dtype).itemsize == 4 else 2048
    cases = [(1, 13), (3, 4 * 3 * 5 + 2), (100, 4 * 100 + 250), (q - 1, 4 * (q - 1) * 2 + 1),
             (q, 4 * q * 3), (q + 1, 4 * (q + 1) + 2 * (q + 1)), (5 * q + 3, 4 * (5 * q + 3) + 7),
             (40 * q, 4 * 40 * q * 2 + 3 * 40 * q + 1), (1000, 1000), (50, 37)]
    for c, (run, n) in enumerate(cases):
        for few in (False, True):
            K = sorted_runs(g, dtype, desc, n, run, few)
            say("merge_runs4", np.dtype(dtype).name, desc, n, run, few)
            got = om.merge_runs4(dev_typed(K), run, descending=desc)
            want = oracle.merge_runs(K, run, 4, descending=desc)
            assert_same(host_bits(got), as_bits(want), "4-way pass (n=%d, run=%d)" % (n, run))


def test_merge_runs4_headline_size():
    """A 4-way pass over 2^28 int32 keys in sorted runs of 2^20 (uniform
    over the int32 range), against the oracle's k-way pass; and the last
    pass of a 2^28 sort (runs of 2^26, one group)."""
    n = 1 << 28
    g = np.random.Generator(np.random.PCG64(811))
    K = g.integers(-(1 << 31), 1 << 31, size=n, dtype=np.int64).astype(np.int32)
    for run in (1 << 20, 1 << 26):
        R = np.sort(K.reshape(-1, run), axis=1).reshape(-1)
        say("merge_runs4 headline size", n, run)
        got = host(om.merge_runs4(dev(R), run))
        assert np.array_equal(got, oracle.merge_runs(R, run, 4)), "run %d" % run
        del got
    torch.cuda.empty_cache()


def test_merge_runs4_unsorted_input_returns():
    """Unsorted runs give an unspecified output but every access stays in
    the arrays (the plan's cells may collide; the cell kernel clamps what it
    reads): the call returns, and the words around the output are intact."""
    g = np.random.Generator(np.random.PCG64(812))
    n = 300001
    K = g.integers(-1000, 1000, size=n).astype(np.int32)
    sentinel = -123456789
    buf = torch.full((n + 64,), sentinel, dtype=torch.int32, device=DEV)
    out = buf[32:32 + n]
    for run in (1, 777, 2048, 65536):
        say("merge_runs4 unsorted", n, run)
        om.merge_runs4(dev(K), run, out=out)
        torch.cuda.synchronize()
        h = host(buf)
        assert np.all(h[:32] == sentinel) and np.all(h[32 + n:] == sentinel), run


def batch_case(g, dtype, desc, pairs, scale):
    la = g.integers(0, scale + 1, size=pairs) * (g.random(pairs) > 0.15)
    lb = g.integers(0, scale + 1, size=pairs) * (g.random(pairs) > 0.15)
    a_off = np.concatenate([[0], np.cumsum(la)]).astype(np.int64)
    b_off = np.concatenate([[0], np.cumsum(lb)]).astype(np.int64)
    A = np.empty(int(a_off[-1]), dtype=dtype)
    B = np.empty(int(b_off[-1]), dtype=dtype)
    for p in range(pairs):
        a, b = typed_pair(g, dtype, desc, int(la[p]), int(lb[p]))
        A[a_off[p]:a_off[p + 1]] = a
        B[b_off[p]:b_off[p + 1]] = b
    return A, a_off, B, b_off


@pytest.mark.parametrize("dtype,desc", [(np.int32, False), (np.float32, True), (np.int64, True),
                                        (np.uint64, False), (np.float64, False)],
                         ids=["int32-asc", "float32-desc", "int64-desc", "uint64-asc",
                              "float64-asc"])
def test_batched_merges(dtype, desc):
    """Batches of 1 to 3000 merges of mixed sizes (empty merges and sides,
    merges shorter and much longer than a segment), keys and pairs."""
    needs_torch_dtype(dtype)
    g = np.random.Generator(np.random.PCG64(760 + [np.int32, np.float32, np.int64, np.uint64,
                                                   np.float64].index(dtype)))
    for pairs, scale in ((1, 90000), (7, 20000), (300, 900), (3000, 40)):
        A, a_off, B, b_off = batch_case(g, dtype, desc, pairs, scale)
        say("batched", np.dtype(dtype).name, desc, pairs, A.size, B.size)
        da, db = dev(a_off), dev(b_off)
        got = om.merge_batched(dev_typed(A), da, dev_typed(B), db, descending=desc)
        want = oracle.merge_batched(A, a_off, B, b_off, descending=desc)
        assert_same(host_bits(got), as_bits(want), "batched keys")
        Av, Bv = tags64(A.size, B.size)
        gk, gv = om.merge_batched(dev_typed(A), da, dev_typed(B), db, dev_typed(Av),
                                  dev_typed(Bv), descending=desc)
        wk, wv = oracle.merge_batched(A, a_off, B, b_off, Av, Bv, descending=desc)
        assert_same(host_bits(gk), as_bits(wk), "batched pair keys")
        assert_same(host_bits(gv), as_bits(wv), "batched pair payloads")


@pytest.mark.parametrize("per_side", [4096, 8192, 16384])
def test_batched_merges_on_segment_multiples(per_side):
    """Batches of equal merges whose starts fall on multiples of the batch
    segment length (16,384 outputs for int32 keys): the plan moves those
    multiples off the merge starts instead of leaving empty segments.  Every
    output, with payloads, against the oracle."""
    g = np.random.Generator(np.random.PCG64(790 + per_side // 4096))
    pairs = (1 << 24) // per_side  # 2^25 outputs: large enough for 16,384-output segments
    a_off = np.arange(pairs + 1, dtype=np.int64) * per_side
    b_off = a_off.copy()
    A = np.sort(g.integers(-(1 << 31), 1 << 31, size=(pairs, per_side)), axis=1)
    B = np.sort(g.integers(-1000, 1000, size=(pairs, per_side)), axis=1)
    A, B = A.astype(np.int32).reshape(-1), B.astype(np.int32).reshape(-1)
    say("batched on segment multiples", per_side, pairs)
    Av, Bv = tags(A.size, B.size)
    gk, gv = om.merge_batched(dev(A), dev(a_off), dev(B), dev(b_off), dev(Av.view(np.int32)),
                              dev(Bv.view(np.int32)))
    wk, wv = oracle.merge_batched(A, a_off, B, b_off, Av, Bv)
    assert_same(host(gk), wk, "keys")
    assert_same(host(gv).view(np.uint32), wv, "payloads")
    got = om.merge_batched(dev(A), dev(a_off), dev(B), dev(b_off))
    assert_same(host(got), wk, "keys only")


def test_batched_invalid_offsets_return():
    """Offsets are device data and are not checked; offsets that break the
    contract (negative, past the ends, decreasing) give an unspecified output
    but the call returns and later work is unaffected (the kernels clamp
    every range; the CPU emulation checks each access of such cases)."""
    g = np.random.Generator(np.random.PCG64(777))
    A = g.integers(0, 50, size=5000).astype(np.int32)
    B = g.integers(0, 50, size=3000).astype(np.int32)
    a_off = g.integers(-(1 << 40), 1 << 40, size=41).astype(np.int64)
    b_off = g.integers(-5, 3005, size=41).astype(np.int64)
    out = om.merge_batched(dev(A), dev(a_off), dev(B), dev(b_off))
    torch.cuda.synchronize()
    assert out.numel() == 8000
    A2, B2 = pair(g, 20000, 10000, 100)
    assert_same(host(om.merge_i32(dev(A2), dev(B2))), oracle.merge_i32(A2, B2), "after")


def test_batched_single_merge_is_merge():
    """A batch of one merge is the plain merge."""
    g = np.random.Generator(np.random.PCG64(771))
    A, B = pair(g, 1 << 22, 3 << 20, 1 << 20)
    got = om.merge_batched(dev(A), dev(np.array([0, A.size], dtype=np.int64)), dev(B),
                           dev(np.array([0, B.size], dtype=np.int64)))
    assert_same(host(got), host(om.merge_i32(dev(A), dev(B))), "batch of one")


# ------------------------------------------------------ beyond 32-bit indices


def test_more_than_2p32_outputs():
    """m = n = 2^31 + 1000 int32 keys (2^32 + 2000 outputs, 32 GiB in HBM),
    built on the device with a closed form: A[i] = i >> 2 and B[j] = j >> 2,
    so the stable merge is C[k] = k >> 3 (each value four times from A, then
    four times from B) and co_rank(k) = 4*(k >> 3) + min(k & 7, 4).  This
    checks every output and sampled co-ranks past 2^31 and 2^32, where 32-bit
    index arithmetic would wrap."""
    m = n = (1 << 31) + 1000
    total = m + n
    say("beyond 2^32", m, n)
    a = (torch.arange(m, dtype=torch.int64, device=DEV) >> 2).to(torch.int32)
    b = (torch.arange(n, dtype=torch.int64, device=DEV) >> 2).to(torch.int32)
    c = om.merge_i32(a, b)
    chunk = 1 << 28
    for k0 in range(0, total, chunk):
        k1 = min(k0 + chunk, total)
        want = (torch.arange(k0, k1, dtype=torch.int64, device=DEV) >> 3).to(torch.int32)
        if not torch.equal(c[k0:k1], want):
            bad = int(torch.nonzero(c[k0:k1] != want)[0, 0]) + k0
            raise AssertionError("beyond 2^32: first difference at %d" % bad)
    ks = torch.tensor([0, 1, 7, 8, (1 << 31) - 3, (1 << 31) + 5, (1 << 32) - 1, 1 << 32,
                       (1 << 32) + 3, total - 1, total], dtype=torch.int64, device=DEV)
    got = om.co_rank(a, b, ks).cpu().numpy()
    kk = ks.cpu().numpy()
    want = 4 * (kk >> 3) + np.minimum(kk & 7, 4)
    want = np.minimum(want, m)
    assert np.array_equal(got, want), (got, want)
    del a, b, c
    torch.cuda.empty_cache()


def test_sort_more_than_2p31_keys():
    """A stable sort of n = 2^31 + 1000 int32 keys with int64 payloads, built
    on the device: key[i] = (n-1-i) >> 2 and payload[i] = i.  Sorted
    ascending, output p holds key p >> 2, and the four equal keys keep their
    input order, so its payload is n - 4 - 4*(p >> 2) + (p & 3)."""
    n = (1 << 31) + 1000
    say("sort beyond 2^31", n)
    i = torch.arange(n, dtype=torch.int64, device=DEV)
    keys = ((n - 1 - i) >> 2).to(torch.int32)
    gk, gv = om.sort(keys, i)
    del keys
    chunk = 1 << 28
    for p0 in range(0, n, chunk):
        p = torch.arange(p0, min(p0 + chunk, n), dtype=torch.int64, device=DEV)
        assert torch.equal(gk[p0:p0 + p.numel()], (p >> 2).to(torch.int32)), p0
        assert torch.equal(gv[p0:p0 + p.numel()], n - 4 - 4 * (p >> 2) + (p & 3)), p0
    del gk, gv, i
    torch.cuda.empty_cache()


# ------------------------------------------------------- full-size workloads

@pytest.mark.parametrize("name", ORDER)
def test_workload_bit_exact(name):
    w = WORKLOADS[name]
    say("workload", name, w.m, w.n)
    arrs = w.make()
    if w.kv:
        Ak, Av, Bk, Bv = arrs
        gk, gv = om.merge_kv(dev(Ak), dev(Av), dev(Bk), dev(Bv))
        gk, gv = host(gk), host(gv).view(np.uint32)
        wk, wv = oracle.merge_kv(Ak, Av, Bk, Bv)
        assert_same(gk, wk, name + " keys")
        assert_same(gv, wv, name + " payloads")
        # merged (key, payload) strictly increasing: the lexicographic sort
        assert np.all((gk[1:] > gk[:-1]) | ((gk[1:] == gk[:-1]) & (gv[1:] > gv[:-1])))
    else:
        A, B = arrs
        got = host(om.merge_i32(dev(A), dev(B)))
        assert_same(got, oracle.merge_i32(A, B), name)
        if name.startswith("even_odd"):
            h = 1 << 22
            assert np.array_equal(got[:h], np.arange(h, dtype=np.int32))


def _check_partition(A, B, part, seg_len):
    """Each boundary's co-rank is the unique split that passes the acceptance
    test A[i-1] <= B[j] and B[j-1] < A[i] (j = k - i), with the usual
    exemptions at the array ends."""
    m, n = A.size, B.size
    ks = np.minimum(np.arange(part.size, dtype=np.int64) * seg_len, m + n)
    I, J = part, ks - part
    assert np.all((I >= np.maximum(0, ks - n)) & (I <= np.minimum(ks, m)))
    A64, B64 = A.astype(np.int64), B.astype(np.int64)
    ok_lo = (I == 0) | (J == n) | (A64[np.clip(I - 1, 0, m - 1)] <= B64[np.clip(J, 0, n - 1)])
    ok_hi = (J == 0) | (I == m) | (B64[np.clip(J - 1, 0, n - 1)] < A64[np.clip(I, 0, m - 1)])
    assert np.all(ok_lo & ok_hi)


@pytest.mark.parametrize("shape", ["clustered", "four_values", "exponential"])
def test_partition_full_size_key_shapes(shape):
    """The partition's probe placement interpolates on the keys and falls
    back to even splits where that fails; at 2^27 + 2^27 keys shaped against
    it (half of A in a tiny range, four distinct values, exponential), every
    boundary must still be the exact co-rank and the merge bit-exact."""
    n = 1 << 27
    g = torch.Generator(device=DEV)
    g.manual_seed(4100 + ["clustered", "four_values", "exponential"].index(shape))
    if shape == "clustered":
        a = torch.cat([torch.randint(0, 1000, (n // 2,), device=DEV, generator=g),
                       torch.randint(10**9, 2 * 10**9, (n // 2,), device=DEV, generator=g)])
        b = torch.randint(0, 2 * 10**9, (n,), device=DEV, generator=g)
    elif shape == "four_values":
        a = torch.randint(0, 4, (n,), device=DEV, generator=g)
        b = torch.randint(0, 4, (n,), device=DEV, generator=g)
    else:
        e = torch.empty(2 * n, dtype=torch.float64, device=DEV).exponential_(1.0, generator=g)
        a, b = (e[:n] * 1e6).to(torch.int64), (e[n:] * 1e6).to(torch.int64)
    a = torch.sort(a.to(torch.int32)).values
    b = torch.sort(b.to(torch.int32)).values
    say("partition key shape", shape, n)
    seg_len = om.segment_length(n, n)
    part = om.partition(a, b, seg_len)
    got = host(om.merge_segments_i32(a, b, part, seg_len))
    A, B = host(a), host(b)
    _check_partition(A, B, host(part), seg_len)
    assert_same(got, oracle.merge_i32(A, B), shape)
    del a, b


def test_headline_stage_path_matches():
    """The launch sequence the benchmark times (partition, then segment
    merge, with the library's own segment length) on the headline workload,
    checked on every output."""
    w = WORKLOADS["uniform_i32_2p28x2p28"]
    A, B = w.make()
    a, b = dev(A), dev(B)
    seg_len = om.segment_length(w.m, w.n)
    say("headline stages", seg_len)
    part = om.partition(a, b, seg_len)
    got = host(om.merge_segments_i32(a, b, part, seg_len))
    _check_partition(A, B, host(part), seg_len)
    assert_same(got, oracle.merge_i32(A, B), "headline")


# ------------------------------------------------------- random mix

def _mix_keys(g, dtype, n):
    """Keys of one of several shapes: four values, the whole range, two
    far-apart clusters, exponential, all equal, small signed."""
    if dtype in (np.float32, np.float64):
        pool = float_pool(dtype)
        return np.ascontiguousarray(pool[g.integers(0, pool.size, size=n)])
    info = np.iinfo(dtype)
    kind = int(g.integers(0, 6))
    if kind == 0:
        x = g.integers(0, 4, size=n)
    elif kind == 1:
        return g.integers(info.min, info.max, size=n, dtype=dtype, endpoint=True)
    elif kind == 2:
        x = np.concatenate([g.integers(0, 50, size=n // 2), g.integers(10**6, 10**7, size=n - n // 2)])
    elif kind == 3:
        x = (g.exponential(1.0, size=n) * 1e5).astype(np.int64)
    elif kind == 4:
        x = np.full(n, 7)
    else:
        x = g.integers(-1000, 1000, size=n)
    if info.min == 0:
        x = np.abs(x)
    return np.ascontiguousarray(x.astype(dtype))


def test_random_mix_against_oracle():
    """500 seeded cases drawn across every entry point (merge, pairs, sort,
    batch), key kind, direction and payload width, with sizes around the
    2048-output tile and up to 10^5, and key shapes that stress the
    partition's probe placement; every output against the oracle."""
    g = np.random.Generator(np.random.PCG64(8080))
    done = 0
    while done < 500:
        dtype, desc = TYPED[int(g.integers(0, len(TYPED)))]
        if np.dtype(dtype) == np.uint64 and not hasattr(torch, "uint64"):
            continue
        if np.dtype(dtype) == np.uint32 and not hasattr(torch, "uint32"):
            continue
        what = int(g.integers(0, 3))
        m = int(g.choice([0, 1, 2047, 2048, 2049, int(g.integers(1, 100000))]))
        n = int(g.choice([0, 1, 2047, 2048, 2049, int(g.integers(1, 100000))]))
        vdt = [None, np.uint32, np.int64][int(g.integers(0, 3))]
        say("mix", done, what, np.dtype(dtype).name, desc, m, n, vdt)
        if what == 0:
            A = oracle.sort(_mix_keys(g, dtype, m), descending=desc)
            B = oracle.sort(_mix_keys(g, dtype, n), descending=desc)
            if vdt is None:
                got = om.merge(dev_typed(A), dev_typed(B), descending=desc)
                assert_same(host_bits(got), as_bits(oracle.merge_keys(A, B, descending=desc)), "mix merge")
            else:
                Av, Bv = (np.arange(m) * 3 + 1).astype(vdt), (np.arange(n) * 5 + 2).astype(vdt)
                gk, gv = om.merge_pairs(dev_typed(A), dev_typed(Av), dev_typed(B), dev_typed(Bv),
                                        descending=desc)
                wk, wv = oracle.merge_pairs(A, Av, B, Bv, descending=desc)
                assert_same(host_bits(gk), as_bits(wk), "mix pair keys")
                assert_same(host_bits(gv), as_bits(wv), "mix pair payloads")
        elif what == 1:
            K = _mix_keys(g, dtype, m)
            if vdt is None:
                got = om.sort(dev_typed(K), descending=desc)
                assert_same(host_bits(got), as_bits(oracle.sort(K, descending=desc)), "mix sort")
            else:
                V = (np.arange(m) * 7 + 3).astype(vdt)
                gk, gv = om.sort(dev_typed(K), dev_typed(V), descending=desc)
                wk, wv = oracle.sort(K, V, descending=desc)
                assert_same(host_bits(gk), as_bits(wk), "mix sort keys")
                assert_same(host_bits(gv), as_bits(wv), "mix sort payloads")
        else:
            pairs = int(g.choice([1, 3, 50, 1000]))
            scale = int(g.choice([3, 100, 5000]))
            la = g.integers(0, scale + 1, size=pairs)
            lb = g.integers(0, scale + 1, size=pairs)
            ao = np.concatenate([[0], np.cumsum(la)]).astype(np.int64)
            bo = np.concatenate([[0], np.cumsum(lb)]).astype(np.int64)
            A = np.concatenate([oracle.sort(_mix_keys(g, dtype, int(x)), descending=desc) for x in la])
            B = np.concatenate([oracle.sort(_mix_keys(g, dtype, int(x)), descending=desc) for x in lb])
            A, B = np.ascontiguousarray(A.astype(dtype)), np.ascontiguousarray(B.astype(dtype))
            got = om.merge_batched(dev_typed(A), torch.from_numpy(ao).to(DEV), dev_typed(B),
                                   torch.from_numpy(bo).to(DEV), descending=desc)
            want = oracle.merge_batched(A, ao, B, bo, descending=desc)
            assert_same(host_bits(got), as_bits(want), "mix batch")
        done += 1

"""Runs the CPU emulation of the HIP kernels (libemu.so, built with ASan and
UBSan) on seeded cases and compares every output with the oracle.

Started by tests/test_kernel_emulation.py in a child process whose
LD_PRELOAD holds the sanitizer runtime; any out-of-bounds or misaligned
access aborts the child.  Exit status 0 = every case matched.

usage: run_emu_cases.py LIBEMU GROUP
"""
import ctypes
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path[:0] = [os.path.dirname(os.path.dirname(HERE))]
import oracle  # noqa: E402

U31 = np.uint32(1 << 31)


def load(path):
    lib = ctypes.CDLL(path)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.emu_tile.argtypes = [i32, i32]
    lib.emu_tile.restype = i32
    lib.emu_partition.argtypes = [i32, p, i64, p, i64, i64, p]
    lib.emu_co_rank.argtypes = [p, i64, p, i64, p, i64, p]
    lib.emu_merge_i32.argtypes = [i32, p, i64, p, i64, p, i64, p]
    lib.emu_merge_kv.argtypes = [i32, p, p, i64, p, p, i64, p, i64, p, p]
    lib.emu_direct.argtypes = [p, i64, p, i64, p, i64, i32]
    lib.emu_merge_typed.argtypes = [i32, i32, i32, p, p, i64, p, p, i64, i64, p, p, p]
    lib.emu_merge_typed.restype = i32
    lib.emu_sort.argtypes = [i32, i32, i32, p, p, i64, p, p, i64]
    lib.emu_sort.restype = i32
    lib.emu_batched.argtypes = [i32, i32, i32, p, p, p, i64, p, p, p, i64, i64, i64, p, p]
    lib.emu_batched.restype = i32
    lib.emu_typed_tile.argtypes = [i32, i32, i32]
    lib.emu_typed_tile.restype = i32
    lib.emu_sort_tile.argtypes = [i32, i32, i32]
    lib.emu_sort_tile.restype = i32
    lib.emu_merge_runs4.argtypes = [i32, i32, p, i64, i64, p, ctypes.c_uint64]
    lib.emu_merge_runs4.restype = i32
    return lib


def placed(x, off):
    """Copy of x whose data pointer is `off` 4-byte words past a 64-byte
    boundary, so every address phase is exercised."""
    buf = np.empty(x.size + 32, dtype=x.dtype)
    base = (-(buf.ctypes.data // 4)) % 16
    v = buf[base + off: base + off + x.size]
    v[...] = x
    return v


def placed_bytes(x, off):
    """Copy of x (any element size) whose data starts `off` bytes past a
    64-byte boundary (off a multiple of the element size)."""
    raw = np.empty(x.nbytes + 128, dtype=np.uint8)
    start = (-raw.ctypes.data) % 64 + off
    v = raw[start:start + x.nbytes].view(x.dtype)
    v[...] = x
    return v


def ptr(x):
    return ctypes.c_void_p(x.ctypes.data) if x.size else ctypes.c_void_p(0)


def sorted_pair(g, m, n, span):
    """Sorted A (m) and B (n) drawn from one shared value window of `span`
    values, so small spans give many ties across the two arrays."""
    if span >= 1 << 32:
        lo, hi = -(1 << 31), 1 << 31
    else:
        lo = int(g.integers(-(1 << 31), (1 << 31) - span))
        hi = lo + span
    A = np.sort(g.integers(lo, hi, size=m, dtype=np.int64)).astype(np.int32)
    B = np.sort(g.integers(lo, hi, size=n, dtype=np.int64)).astype(np.int32)
    return A, B


class Runner:
    def __init__(self, lib):
        self.lib = lib
        self.fail = 0
        self.cases = 0

    def check(self, ok, what):
        self.cases += 1
        if not ok:
            self.fail += 1
            print("MISMATCH", what, flush=True)

    def partition(self, A, B, seg_len, agree=True, widths=(1, 4, 8, 16, 64, 416)):
        """Partition with each search width; on sorted input all must agree
        (on unsorted input the co-rank is unspecified)."""
        count = (A.size + B.size + seg_len - 1) // seg_len + 1
        got = None
        for lanes in widths:
            part = np.full(count, -7, dtype=np.int64)
            self.lib.emu_partition(lanes, ptr(A), A.size, ptr(B), B.size, seg_len, ptr(part))
            if got is None:
                got = part
            elif agree:
                self.check(np.array_equal(part, got), ("partition width", lanes, A.size, B.size, seg_len))
        return got

    def case_i32(self, variant, A, B, seg_len, offs=(0, 0, 0), label=""):
        m, n = A.size, B.size
        Ap, Bp = placed(A, offs[0]), placed(B, offs[1])
        # variants | 2 do not read the partition: one width checks it
        part = self.partition(Ap, Bp, seg_len, widths=(416,) if variant & 2 else
                              (1, 4, 8, 16, 64, 416))
        I = oracle.co_rank_all(A, B)
        ks = np.minimum(np.arange(part.size, dtype=np.int64) * seg_len, m + n)
        self.check(np.array_equal(part, I[ks]), ("partition", label, m, n, seg_len))
        C = placed(np.full(m + n, 12345, dtype=np.int32), offs[2])
        if m + n:
            self.lib.emu_merge_i32(variant, ptr(Ap), m, ptr(Bp), n, ptr(part), seg_len, ptr(C))
        want = oracle.merge_i32(A, B)
        ok = np.array_equal(C, want)
        if not ok:
            bad = int(np.argmax(C != want))
            label = (label, "first diff", bad, int(C[bad]), int(want[bad]))
        self.check(ok, ("merge_i32", variant, label, m, n, seg_len, offs))

    def case_kv(self, variant, A, B, seg_len, offs=(0, 0, 0, 0, 0, 0), label=""):
        m, n = A.size, B.size
        Av = np.arange(m, dtype=np.uint32)
        Bv = (U31 + np.arange(n, dtype=np.uint32)).astype(np.uint32)
        Ap, Avp, Bp, Bvp = placed(A, offs[0]), placed(Av, offs[1]), placed(B, offs[2]), placed(Bv, offs[3])
        part = self.partition(Ap, Bp, seg_len, widths=(1,))
        Ck = placed(np.zeros(m + n, dtype=np.int32), offs[4])
        Cv = placed(np.zeros(m + n, dtype=np.uint32), offs[5])
        if m + n:
            self.lib.emu_merge_kv(variant, ptr(Ap), ptr(Avp), m, ptr(Bp), ptr(Bvp), n,
                                  ptr(part), seg_len, ptr(Ck), ptr(Cv))
        wk, wv = oracle.merge_kv(A, Av, B, Bv)
        self.check(np.array_equal(Ck, wk) and np.array_equal(Cv, wv),
                   ("merge_kv", variant, label, m, n, seg_len, offs))

    def case_co_rank(self, A, B):
        ks = np.arange(A.size + B.size + 1, dtype=np.int64)
        out = np.zeros_like(ks)
        self.lib.emu_co_rank(ptr(A), A.size, ptr(B), B.size, ptr(ks), ks.size, ptr(out))
        self.check(np.array_equal(out, oracle.co_rank_all(A, B)), ("co_rank", A.size, B.size))


def small_cases(r, g):
    """The seeded cases of the small shapes: (case, A, B, seg_len, offsets)."""
    tile = r.lib.emu_tile(1, 0)
    for c in range(36):
        m, n = (int(x) for x in g.integers(0, 2500, size=2))
        if c % 10 == 0:
            m = 0
        if c % 10 == 1:
            n = 0
        span = int(g.choice([2, 16, 1000, 1 << 32]))
        A, B = sorted_pair(g, m, n, span)
        seg_len = int(g.choice([tile, 2 * tile, 3 * tile, 4 * int(g.integers(1, 300))]))
        offs = tuple(int(x) for x in g.integers(0, 4, size=6))
        yield c, A, B, seg_len, offs


def group_small(r, g):
    """64-lane, 4-item shapes (tile 256): many ring wraps on small inputs."""
    for c, A, B, seg_len, offs in small_cases(r, g):
        r.case_i32(1, A, B, seg_len, offs[:3], "small")
        r.case_kv(1, A, B, seg_len, offs, "small")
        if A.size + B.size <= 400:
            r.case_co_rank(A, B)


def group_small_self(r, g):
    """The same cases (every other one, empty sides included) with each
    workgroup finding its own boundaries."""
    for c, A, B, seg_len, offs in small_cases(r, g):
        if c % 2 == 0:
            r.case_i32(3, A, B, seg_len, offs[:3], "small-self")
            r.case_kv(3, A, B, seg_len, offs, "small-self")


def group_skew(r, g):
    """One side dense, the other packed in a narrow interval: tiles swing
    between all-A and mostly-B, and one ring drains while the other fills."""
    tile = r.lib.emu_tile(1, 0)
    for c in range(12):
        m = int(g.integers(2000, 6000))
        n = int(g.integers(0, 600))
        A = np.sort(g.integers(0, 1 << 20, size=m)).astype(np.int32)
        lo = int(g.integers(0, 1 << 20))
        B = np.sort(g.integers(lo, lo + 64, size=n)).astype(np.int32)
        if c % 2:
            A, B = B, A
        seg_len = int(g.choice([tile, 5 * tile, 4 * int(g.integers(1, 700))]))
        r.case_i32(1, A, B, seg_len, tuple(int(x) for x in g.integers(0, 4, size=3)), "skew")
        r.case_kv(1, A, B, seg_len, tuple(int(x) for x in g.integers(0, 4, size=6)), "skew")


def group_blocks(r, g):
    """Runs of one side longer than a tile: whole tiles come from A alone or
    B alone (the one-sided fast path), with mixed tiles at the seams."""
    tile = r.lib.emu_tile(1, 0)
    cases = []
    for c in range(10):
        L = [int(x) for x in g.integers(1, 6 * tile, size=int(g.integers(2, 7)))]
        A, B, v = [], [], 0
        for i, ln in enumerate(L):
            tgt = A if (i + c) % 2 == 0 else B
            tgt.extend(range(v, v + ln))
            v += ln - (2 if c % 3 == 0 else 0)  # seams with equal keys across sides
        A = np.array(A, dtype=np.int32); B = np.array(B, dtype=np.int32)
        A.sort(); B.sort()
        cases.append((A, B))
    cases.append((np.arange(0, 3000, dtype=np.int32), np.arange(3000, 5000, dtype=np.int32)))
    cases.append((np.arange(3000, 5000, dtype=np.int32), np.arange(0, 3000, dtype=np.int32)))
    cases.append((np.full(2000, 7, np.int32), np.full(3000, 7, np.int32)))
    for A, B in cases:
        seg_len = int(g.choice([tile, 3 * tile, 4 * int(g.integers(1, 700))]))
        r.case_i32(1, A, B, seg_len, tuple(int(x) for x in g.integers(0, 4, size=3)), "blocks")
        r.case_kv(1, A, B, seg_len, tuple(int(x) for x in g.integers(0, 4, size=6)), "blocks")
    tile0 = r.lib.emu_tile(0, 0)
    A = np.arange(0, 9000, dtype=np.int32); B = np.arange(9000, 20000, dtype=np.int32)
    r.case_i32(0, A, B, 3 * tile0, (1, 2, 3), "blocks-prod")
    r.case_kv(0, B, A, 3 * r.lib.emu_tile(0, 1), (0, 1, 2, 3, 1, 2), "blocks-prod")


def group_production(r, g):
    """The shapes the library launches (256 lanes; 2048-output tiles for
    keys alone and for key+payload), over several tiles and segments, and
    over segments shorter than one tile."""
    for kv in (False, True):
        tile = r.lib.emu_tile(0, int(kv))
        for c in range(4):
            m = int(g.integers(0, 7 * tile))
            n = int(g.integers(0, 7 * tile))
            span = int(g.choice([4, 300, 1 << 32]))
            A, B = sorted_pair(g, m, n, span)
            seg_len = [tile, 3 * tile, 2 * tile + 1364, 4 * tile][c]
            # partition array, or boundaries found by each workgroup (every
            # other segment length)
            for variant in ((0, 2) if c % 2 == 0 else (0,)):
                if kv:
                    r.case_kv(variant, A, B, seg_len,
                              tuple(int(x) for x in g.integers(0, 4, size=6)), "prod")
                else:
                    r.case_i32(variant, A, B, seg_len,
                               tuple(int(x) for x in g.integers(0, 4, size=3)), "prod")
        # segments shorter than one tile: each workgroup's only tile is short
        for seg_len in (4, 12):
            m, n = int(g.integers(0, 300)), int(g.integers(1, 300))
            A, B = sorted_pair(g, m, n, 300)
            for c_off in (0, 3):  # aligned outputs (register stores) and staged ones
                for variant in ((0, 2) if seg_len == 12 and c_off == 0 else (0,)):
                    if kv:
                        r.case_kv(variant, A, B, seg_len, (0, 1, 2, 3, c_off, c_off), "prod-short")
                    else:
                        r.case_i32(variant, A, B, seg_len, (1, 2, c_off), "prod-short")


def group_search(r, g):
    """Key distributions chosen against the partition's interpolated probe
    placement: clustered, exponential, two-valued, all equal, nearly linear
    with jumps, and the int32 extremes.  Partitions at every search width
    against the oracle's co-ranks (exact whatever the placement)."""
    n0 = 60000
    lo32, hi32 = -(1 << 31), (1 << 31) - 1
    cases = [
        ("clustered", np.concatenate([g.integers(0, 1000, n0 // 2), g.integers(10**9, 2 * 10**9, n0 // 2)]),
         g.integers(0, 2 * 10**9, n0)),
        ("exponential", (g.exponential(1.0, n0) * 1e6).astype(np.int64),
         (g.exponential(1.0, n0 // 3) * 1e6).astype(np.int64)),
        ("two-valued", g.integers(0, 2, n0), g.integers(0, 2, n0 // 2)),
        ("all equal", np.full(n0, 5), np.full(n0 // 4, 5)),
        ("linear with jumps", 3 * np.arange(n0) + 1000 * (np.arange(n0) > n0 // 3),
         3 * np.arange(n0) + 1 + 10**6 * (np.arange(n0) > 2 * n0 // 3)),
        ("extremes", g.choice([lo32, lo32 + 1, -1, 0, 1, hi32 - 1, hi32], n0),
         g.integers(lo32, hi32, n0, endpoint=True)),
        ("one huge gap", np.concatenate([np.arange(n0 // 2), hi32 - np.arange(n0 // 2)[::-1]]),
         g.integers(0, n0, n0)),
    ]
    for c, (label, A, B) in enumerate(cases):
        A = np.sort(np.asarray(A, dtype=np.int64)).astype(np.int32)
        B = np.sort(np.asarray(B, dtype=np.int64)).astype(np.int32)
        if c % 2:
            A, B = B, A
        seg_len = int(g.choice([389, 1000, 4096]))
        part = r.partition(A, B, seg_len, widths=(416, 4, 1, 8, 64))
        I = oracle.co_rank_all(A, B)
        ks = np.minimum(np.arange(part.size, dtype=np.int64) * seg_len, A.size + B.size)
        r.check(np.array_equal(part, I[ks]), ("search", label, A.size, B.size, seg_len))


def group_unsorted(r, g):
    """Unsorted input breaks the precondition: the kernels must still stop
    and stay inside the arrays (the sanitizers watch every access)."""
    tile = r.lib.emu_tile(1, 0)
    for c in range(15):
        m, n = (int(x) for x in g.integers(0, 1500, size=2))
        A = g.integers(-50, 50, size=m).astype(np.int32)
        B = g.integers(-50, 50, size=n).astype(np.int32)
        seg_len = int(g.choice([tile, 3 * tile, 4 * int(g.integers(1, 200))]))
        part = r.partition(A, B, seg_len, agree=False)
        C = np.zeros(m + n, dtype=np.int32)
        if m + n:
            r.lib.emu_merge_i32(1, ptr(A), m, ptr(B), n, ptr(part), seg_len, ptr(C))
        # a nonsense partition must not take the kernel out of bounds either
        junk = g.integers(-(1 << 40), 1 << 40, size=part.size).astype(np.int64)
        if m + n:
            r.lib.emu_merge_i32(1, ptr(A), m, ptr(B), n, ptr(junk), seg_len, ptr(C))
        r.cases += 1


def group_direct(r, g):
    """The global-memory kernels (basic: two searches; walk: one search)."""
    for c in range(16):
        m, n = (int(x) for x in g.integers(0, 3000, size=2))
        A, B = sorted_pair(g, m, n, int(g.choice([2, 50, 1 << 32])))
        want = oracle.merge_i32(A, B)
        for per in (1, 4, 16, 64, 256):
            for two in (0, 1):
                C = np.full(m + n, 777, dtype=np.int32)
                if m + n:
                    r.lib.emu_direct(ptr(A), m, ptr(B), n, ptr(C), per, two)
                r.check(np.array_equal(C, want), ("direct", m, n, per, two))


KIND_DTYPE = {0: np.int32, 1: np.uint32, 2: np.float32, 3: np.int64, 4: np.uint64,
              5: np.float64}


def float_pool(g, dtype):
    """Special values (signed zeros, infinities, subnormals, NaNs of both
    signs) and random bit patterns of a float dtype, sorted with the oracle's
    totalOrder relation."""
    import functools
    if dtype == np.float32:
        special = np.array([0xFFC00000, 0xFFFFFFFF, 0xFF800001, 0xFF800000, 0xFF7FFFFF,
                            0xBF800000, 0x80000001, 0x80000000, 0x00000000, 0x00000001,
                            0x3F800000, 0x7F7FFFFF, 0x7F800000, 0x7F800001, 0x7FC00000,
                            0x7FFFFFFF], dtype=np.uint32)
        rnd = g.integers(0, 1 << 32, size=80, dtype=np.uint64).astype(np.uint32)
    else:
        special = np.array([0xFFF8000000000000, 0xFFFFFFFFFFFFFFFF, 0xFFF0000000000001,
                            0xFFF0000000000000, 0xFFEFFFFFFFFFFFFF, 0xBFF0000000000000,
                            0x8000000000000001, 0x8000000000000000, 0x0000000000000000,
                            0x0000000000000001, 0x3FF0000000000000, 0x3FF0000000000001,
                            0x7FEFFFFFFFFFFFFF, 0x7FF0000000000000, 0x7FF0000000000001,
                            0x7FF8000000000000, 0x7FFFFFFFFFFFFFFF], dtype=np.uint64)
        rnd = g.integers(0, 1 << 64, size=80, dtype=np.uint64, endpoint=False)
    vals = np.unique(np.concatenate([special, rnd])).view(dtype)

    def cmp(x, y):
        if not oracle.key_le(dtype, x, y):
            return 1
        return 0 if oracle.key_le(dtype, y, x) else -1
    return np.array(sorted(vals.tolist(), key=functools.cmp_to_key(
        lambda a, b: cmp(dtype(a), dtype(b)))), dtype=dtype)


def typed_sorted_pair(g, dtype, desc, m, n, pools):
    """Sorted A, B of one key type in the given direction.  Float keys are
    drawn from pools[dtype], already in IEEE totalOrder."""
    if dtype in (np.float32, np.float64):
        pool = pools[dtype]
        A = pool[np.sort(g.integers(0, len(pool), size=m))]
        B = pool[np.sort(g.integers(0, len(pool), size=n))]
    else:
        info = np.iinfo(dtype)
        wide = np.dtype(dtype).itemsize == 8
        span = int(g.choice([3, 1000, 1 << 40 if wide else 1 << 32]))
        if span > 1000:
            A = np.sort(g.integers(info.min, info.max, size=m, dtype=dtype, endpoint=True))
            B = np.sort(g.integers(info.min, info.max, size=n, dtype=dtype, endpoint=True))
        else:
            lo = int(g.integers(info.min, int(info.max) - span, dtype=dtype))
            A = np.sort(g.integers(lo, lo + span, size=m, dtype=dtype))
            B = np.sort(g.integers(lo, lo + span, size=n, dtype=dtype))
    if desc:
        A, B = A[::-1], B[::-1]
    return np.ascontiguousarray(A), np.ascontiguousarray(B)


def group_orders(r, g):
    """Every key order (int32/uint32/float32/int64/uint64/float64, ascending
    and descending) and payload width the emulation library holds, through
    the ordered partition and merge kernels, against the oracle; the
    partition against co-ranks read off the oracle's payload tags."""
    pools = {np.float32: float_pool(g, np.float32), np.float64: float_pool(g, np.float64)}
    plan = []
    for order in (0, 1, 2, 3, 4, 5, 8, 9, 10, 11, 12, 13):
        for vw in (0, 1, 2):
            # 1 | 2 and 0 | 2: the same shapes, each workgroup finding its own
            # boundaries (on a spread of 4- and 8-byte orders)
            self_variants = (3, 2) if order in (0, 10, 11, 13) else ()
            for variant in (1, 0) + self_variants:
                plan.append((order, vw, variant))
    ran = 0
    for c, (order, vw, variant) in enumerate(plan):
        dtype = KIND_DTYPE[order & 7]
        desc = bool(order & 8)
        tile = r.lib.emu_typed_tile(variant & 1, order, vw)
        for rep in range(3 if variant == 1 else 1):
            m, n = (int(x) for x in g.integers(0, 5 * tile, size=2))
            if rep == 2:
                m = 0
            A, B = typed_sorted_pair(g, dtype, desc, m, n, pools)
            vdt = np.uint64 if vw == 2 else np.uint32
            top = vdt(1 << (63 if vw == 2 else 31))
            Av = np.arange(m, dtype=vdt)
            Bv = (top + np.arange(n, dtype=vdt)).astype(vdt)
            wk, wv = oracle.merge_pairs(A, Av, B, Bv, desc)
            from_a = np.concatenate([[0], np.cumsum(wv < top)]).astype(np.int64)
            seg_len = int(g.choice([tile, 3 * tile, 4 * int(g.integers(1, 300))]))
            count = (m + n + seg_len - 1) // seg_len + 1
            part = np.full(count, -3, dtype=np.int64)
            Ck = np.zeros(m + n, dtype=A.dtype)
            Cv = np.zeros(m + n, dtype=vdt)
            held = r.lib.emu_merge_typed(variant, order, vw, ptr(A), ptr(Av) if vw else None, m,
                                         ptr(B), ptr(Bv) if vw else None, n, seg_len, ptr(part),
                                         ptr(Ck), ptr(Cv) if vw else None)
            if not held:
                break
            ran += 1
            ks = np.minimum(np.arange(count, dtype=np.int64) * seg_len, m + n)
            r.check(np.array_equal(part, from_a[ks]), ("typed partition", order, vw, m, n, seg_len))
            ok = np.array_equal(Ck.view(np.uint8), wk.view(np.uint8))
            if vw:
                ok = ok and np.array_equal(Cv, wv)
            r.check(ok, ("typed merge", order, vw, variant, m, n, seg_len))
    r.check(ran >= 40, ("typed combinations run", ran))


SORT_COMBOS = [(1, 0, 0), (1, 0, 2), (1, 10, 1), (1, 3, 2), (1, 13, 0), (0, 0, 0), (0, 0, 2),
               (0, 13, 1), (0, 11, 0)]


def unsorted_keys(g, dtype, n, pools):
    """Unsorted keys with many ties (integers) or specials (floats)."""
    if dtype in (np.float32, np.float64):
        pool = pools[dtype]
        return pool[g.integers(0, min(len(pool), int(g.choice([5, len(pool)]))), size=n)]
    info = np.iinfo(dtype)
    if g.random() < 0.5:
        return g.integers(-3 if info.min < 0 else 0, 4, size=n).astype(dtype)
    return g.integers(info.min, info.max, size=n, dtype=dtype, endpoint=True)


MULTIWAY_COMBOS = [(1, 0), (1, 1), (1, 10), (1, 11), (1, 13), (0, 0), (0, 13)]


def group_sort(r, g):
    """The merge sort (block sort, then plan + descriptor merges per pass)
    against the oracle's stable sort: sizes around tile multiples, several
    segment lengths (many segments per pair, or one), in place and not."""
    pools = {np.float32: float_pool(g, np.float32), np.float64: float_pool(g, np.float64)}
    for variant, order, vw in SORT_COMBOS:
        dtype = KIND_DTYPE[order & 7]
        desc = bool(order & 8)
        tile = r.lib.emu_sort_tile(variant, order, vw)  # the block sort's runs
        sizes = [0, 1, 5, tile - 1, tile, tile + 1, 2 * tile + 3] + \
            [int(x) for x in g.integers(3 * tile, 9 * tile if variant else 4 * tile,
                                        size=2 if variant else 1)]
        for c, n in enumerate(sizes):
            K = np.ascontiguousarray(unsorted_keys(g, dtype, n, pools))
            vdt = np.uint64 if vw == 2 else np.uint32
            V = (np.arange(n, dtype=vdt) * vdt(3) + vdt(1)).astype(vdt)
            seg_len = int(g.choice([tile, 3 * tile, 9 * tile, 100, 4 * int(g.integers(1, 200))]))
            in_place = c % 3 == 2
            outk = K.copy() if in_place else np.zeros_like(K)
            outv = V.copy() if in_place else np.zeros_like(V)
            src_k = outk if in_place else K
            src_v = outv if in_place else V
            held = r.lib.emu_sort(variant, order, vw, ptr(src_k), ptr(src_v) if vw else None, n,
                                  ptr(outk), ptr(outv) if vw else None, seg_len)
            r.check(held == 1, ("sort combo held", variant, order, vw))
            if vw:
                wk, wv = oracle.sort(K, V, descending=desc)
                ok = np.array_equal(outk.view(np.uint8), wk.view(np.uint8)) and \
                    np.array_equal(outv, wv)
            else:
                wk = oracle.sort(K, descending=desc)
                ok = np.array_equal(outk.view(np.uint8), wk.view(np.uint8))
            r.check(ok, ("sort", variant, order, vw, n, seg_len, in_place))


def group_batched(r, g):
    """Batches of merges (empty merges and sides, tiny and multi-segment
    merges, merges much longer than a segment) against the oracle."""
    pools = {np.float32: float_pool(g, np.float32), np.float64: float_pool(g, np.float64)}
    for variant, order, vw in SORT_COMBOS:
        dtype = KIND_DTYPE[order & 7]
        desc = bool(order & 8)
        tile = r.lib.emu_typed_tile(variant, order, vw)
        for c in range(5 if variant else 2):
            pairs = int(g.choice([1, 3, 40, 300, 2000]))
            scale = int(g.choice([3, tile // 2, 3 * tile])) if pairs < 2000 else 3
            empty = 0.15 if c % 3 else 0.7  # many empty merges: tiles overflow their piece list
            la = g.integers(0, scale + 1, size=pairs) * (g.random(pairs) > empty)
            lb = g.integers(0, scale + 1, size=pairs) * (g.random(pairs) > empty)
            a_off = np.concatenate([[0], np.cumsum(la)]).astype(np.int64)
            b_off = np.concatenate([[0], np.cumsum(lb)]).astype(np.int64)
            m, n = int(a_off[-1]), int(b_off[-1])
            A = np.empty(m, dtype=dtype)
            B = np.empty(n, dtype=dtype)
            for p in range(pairs):
                a, b = typed_sorted_pair(g, dtype, desc, int(la[p]), int(lb[p]), pools)
                A[a_off[p]:a_off[p + 1]] = a
                B[b_off[p]:b_off[p + 1]] = b
            vdt = np.uint64 if vw == 2 else np.uint32
            top = vdt(1 << (63 if vw == 2 else 31))
            Av = np.arange(m, dtype=vdt)
            Bv = (top + np.arange(n, dtype=vdt)).astype(vdt)
            if vw:
                wk, wv = oracle.merge_batched(A, a_off, B, b_off, Av, Bv, descending=desc)
            else:
                wk = oracle.merge_batched(A, a_off, B, b_off, descending=desc)
            # seg_len 0 = the tile path for short merges
            seg_lens = [int(g.choice([tile, 3 * tile, 100, 4 * int(g.integers(1, 300))])), 0]
            if pairs >= 2000:
                seg_lens = [0]  # thousands of one-workgroup merges: the tile path only
            # the tile path also into an output one element off 16-byte
            # alignment (the staged store instead of the register store)
            runs = [(sl, 0) for sl in seg_lens] + ([(0, 1)] if 0 in seg_lens else [])
            for seg_len, skew in runs:
                Ck = np.zeros(m + n + skew, dtype=dtype)[skew:]
                Cv = np.zeros(m + n, dtype=vdt)
                held = r.lib.emu_batched(variant, order, vw, ptr(A), ptr(Av) if vw else None,
                                         ptr(a_off), m, ptr(B), ptr(Bv) if vw else None,
                                         ptr(b_off), n, pairs, seg_len, ptr(Ck),
                                         ptr(Cv) if vw else None)
                r.check(held == 1, ("batched combo held", variant, order, vw))
                ok = np.array_equal(Ck.view(np.uint8), wk.view(np.uint8))
                if vw:
                    ok = ok and np.array_equal(Cv, wv)
                r.check(ok, ("batched", variant, order, vw, pairs, m, n, seg_len, skew))


def group_batched_aligned(r, g):
    """Batches whose merge starts fall on multiples of the segment length
    (merges of seg_len/2, seg_len and 2*seg_len outputs, some empty): the plan
    moves those multiples off the starts instead of leaving empty segments."""
    for variant in (1, 0):
        tile = r.lib.emu_typed_tile(variant, 0, 0)
        for seg_len in (tile, 2 * tile):
            for per in (seg_len // 2, seg_len, 2 * seg_len):
                pairs = 12
                la = np.full(pairs, per // 2, dtype=np.int64)
                lb = np.full(pairs, per - per // 2, dtype=np.int64)
                la[3] = lb[3] = 0            # an empty merge
                la[5], lb[5] = per, 0        # a merge with no B
                a_off = np.concatenate([[0], np.cumsum(la)]).astype(np.int64)
                b_off = np.concatenate([[0], np.cumsum(lb)]).astype(np.int64)
                m, n = int(a_off[-1]), int(b_off[-1])
                A = np.empty(m, dtype=np.int32)
                B = np.empty(n, dtype=np.int32)
                for q in range(pairs):
                    a, b = sorted_pair(g, int(la[q]), int(lb[q]), int(g.choice([3, 1 << 32])))
                    A[a_off[q]:a_off[q + 1]] = a
                    B[b_off[q]:b_off[q + 1]] = b
                wk = oracle.merge_batched(A, a_off, B, b_off)
                Ck = np.zeros(m + n, dtype=np.int32)
                held = r.lib.emu_batched(variant, 0, 0, ptr(A), None, ptr(a_off), m, ptr(B), None,
                                         ptr(b_off), n, pairs, seg_len, ptr(Ck), None)
                r.check(held == 1, ("batched combo held", variant))
                r.check(np.array_equal(Ck, wk), ("batched aligned", variant, seg_len, per))


def group_batched_garbage(r, g):
    """Offsets that break the contract (negative, past the ends, decreasing,
    huge) and unsorted keys: the plan and merge kernels must still stay inside
    every array (the sanitizers watch each access) and return."""
    for c in range(12):
        variant, order, vw = SORT_COMBOS[c % len(SORT_COMBOS)]
        dtype = KIND_DTYPE[order & 7]
        pairs = int(g.integers(1, 60))
        m, n = (int(x) for x in g.integers(0, 3000, size=2))
        a_off = g.integers(-(1 << 40), 1 << 40, size=pairs + 1).astype(np.int64)
        b_off = g.integers(-5, n + 5, size=pairs + 1).astype(np.int64)
        if c % 3 == 0:
            a_off = np.sort(g.integers(-3, m + 3, size=pairs + 1)).astype(np.int64)
        A = g.integers(0, 50, size=m).astype(dtype)
        B = g.integers(0, 50, size=n).astype(dtype)
        vdt = np.uint64 if vw == 2 else np.uint32
        Av = np.arange(m, dtype=vdt)
        Bv = np.arange(n, dtype=vdt)
        Ck = np.zeros(m + n, dtype=dtype)
        Cv = np.zeros(m + n, dtype=vdt)
        for seg_len in (int(g.choice([100, 512, 4 * int(g.integers(1, 300))])), 0):
            r.lib.emu_batched(variant, order, vw, ptr(A), ptr(Av) if vw else None, ptr(a_off), m,
                              ptr(B), ptr(Bv) if vw else None, ptr(b_off), n, pairs, seg_len,
                              ptr(Ck), ptr(Cv) if vw else None)
            r.cases += 1


def sorted_runs(g, dtype, n, run, desc, pools):
    """n keys of dtype whose consecutive runs of `run` are each sorted in the
    key order (the oracle's stable sort of each run)."""
    K = np.ascontiguousarray(unsorted_keys(g, dtype, n, pools))
    for s0 in range(0, n, run):
        K[s0:s0 + run] = oracle.sort(K[s0:s0 + run], descending=desc)
    return K


def group_multiway(r, g):
    """One 4-way pass (plan + cell merges) against the oracle's k-way pass:
    run lengths below, at and around the cell bound q, several groups and a
    ragged last group (one to four runs, a short last run), keys with many
    ties or spread over the type's range, every address phase of the source
    and the output.  The plan's invariants (windows inside runs, at most q
    elements of each pair per cell, outputs consecutive) are checked before
    the merges run."""
    pools = {np.float32: float_pool(g, np.float32), np.float64: float_pool(g, np.float64)}
    for variant, order in MULTIWAY_COMBOS:
        dtype = KIND_DTYPE[order & 7]
        desc = bool(order & 8)
        q = 128 if variant else (4096 if np.dtype(dtype).itemsize == 4 else 2048)
        # long runs put tens of sample points on each side of a group, so
        # the plan's second phase (searches between searched neighbours)
        # runs, across side and group boundaries too
        runs = [1, 3, q // 2, q - 1, q, q + 1, 2 * q, 3 * q + 5, 12 * q + 7, 20 * q] if variant \
            else [q // 2 + 3, 2 * q, 3 * q - 1, 9 * q + 1]
        for c, run in enumerate(runs):
            groups = int(g.integers(1, 4 if variant else 2))
            extra = int(g.integers(0, 4 * run))  # a ragged last group
            n = groups * 4 * run + (extra if c % 2 else 0)
            K = sorted_runs(g, dtype, n, run, desc, pools)
            size = np.dtype(dtype).itemsize
            src = placed_bytes(K, 4 * int(g.integers(0, 4)) // size * size)
            out = placed_bytes(np.zeros_like(K), 4 * int(g.integers(0, 4)) // size * size)
            held = r.lib.emu_merge_runs4(variant, order, ptr(src), n, run, ptr(out), 0)
            r.check(held == 1, ("multiway plan invariants", variant, order, n, run))
            if held == 1:
                want = oracle.merge_runs(K, run, 4, descending=desc)
                r.check(np.array_equal(out.view(np.uint8), want.view(np.uint8)),
                        ("multiway", variant, order, n, run))


def group_multiway_garbage(r, g):
    """The 4-way pass on unsorted runs, with the cell array starting as
    pseudo-random words: the output is unspecified, but the sanitizers see
    no access outside the arrays, and the words around the output stay
    untouched."""
    for variant, order in MULTIWAY_COMBOS:
        dtype = KIND_DTYPE[order & 7]
        size = np.dtype(dtype).itemsize
        q = 128 if variant else (4096 if size == 4 else 2048)
        for run in ([1, 5, q - 1, 3 * q + 1, 20 * q] if variant else [q + 1, 9 * q]):
            n = int(g.integers(1, 4 * run + 1)) + 4 * run * int(g.integers(0, 3))
            K = np.ascontiguousarray(g.integers(-50, 50, size=n).astype(dtype))
            pad = 8
            buf = np.full(n + 2 * pad, 99, dtype=dtype)
            out = buf[pad:pad + n]
            held = r.lib.emu_merge_runs4(variant, order, ptr(K), n, run, ptr(out),
                                         int(g.integers(1, 1 << 62)))
            r.check(held == 1, ("multiway garbage held", variant, order, n, run))
            r.check(np.all(buf[:pad] == 99) and np.all(buf[pad + n:] == 99),
                    ("multiway garbage writes outside", variant, order, n, run))


GROUPS = {"small_self": group_small_self, "multiway_garbage": group_multiway_garbage, "multiway": group_multiway, "batched_aligned": group_batched_aligned, "search": group_search, "batched_garbage": group_batched_garbage, "sort": group_sort, "batched": group_batched, "orders": group_orders, "small": group_small, "direct": group_direct, "skew": group_skew, "blocks": group_blocks,
          "production": group_production, "unsorted": group_unsorted}

if __name__ == "__main__":
    lib = load(sys.argv[1])
    r = Runner(lib)
    GROUPS[sys.argv[2]](r, np.random.Generator(np.random.PCG64(4242)))
    print("cases", r.cases, "failures", r.fail, flush=True)
    sys.exit(1 if r.fail else 0)

"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with the fact.  ``tests/test_oracle_pins.py`` runs
them against the real oracle; ``tests/test_oracle_mutants.py`` runs them
against copies of the oracle with planted mistakes and expects a failure.

Sources of truth used here:
  * values printed on the pages (golden fixtures under tests/golden/);
  * hand derivation from the definition on tiny inputs;
  * brute force: a stable sort of the tagged concatenation A||B;
  * a library routine that is specified to be this merge (heapq.merge is
    stable and takes the first iterable first on equal keys);
  * a structurally different formula: the rank scatter
    A[i] -> C[i + #{b in B : b < A[i]}],  B[j] -> C[j + #{a in A : a <= B[j]}];
  * closed forms of the even/odd workload;
  * invariants: i+j=k, the co-rank bounds, unit steps, order, permutation.
"""
from __future__ import annotations

import heapq
import itertools
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

U31 = np.uint32(1 << 31)


def load_golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def tags(m: int, n: int):
    """Distinct payload tags: A element i -> i, B element j -> 2^31 + j."""
    return (np.arange(m, dtype=np.uint32),
            (U31 + np.arange(n, dtype=np.uint32)).astype(np.uint32))


def as_i32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.int32)


# ---------------------------------------------------------------- golden pins

def pin_worked_example(orc) -> None:
    """Page-printed co-ranks, thread calls and thread-1 output (12-merge/02)."""
    g = load_golden("worked_example_corank.json")
    A, B = as_i32(g["A"]), as_i32(g["B"])
    I = orc.co_rank_all(A, B)
    for k, i, j in zip(g["boundary_k"], g["boundary_i"], g["boundary_j"]):
        assert I[k] == i, ("co_rank(%d)" % k, int(I[k]), i)
        assert k - I[k] == j
    C = orc.merge_i32(A, B)
    out = g["thread1_output"]
    c0 = out["c_start"]
    assert list(C[c0:c0 + len(out["values"])]) == out["values"]
    ks = g["boundary_k"]
    for call in g["thread_calls"]:
        t = call["thread"]
        k0, k1 = ks[t], ks[t + 1]
        assert call["a_start"] == I[k0] and call["a_len"] == I[k1] - I[k0]
        assert call["b_start"] == k0 - I[k0]
        assert call["b_len"] == (k1 - I[k1]) - (k0 - I[k0])
        assert call["c_start"] == k0
        # Merging the thread's two sub-arrays alone gives its slice of C.
        part = orc.merge_i32(A[call["a_start"]:call["a_start"] + call["a_len"]],
                             B[call["b_start"]:call["b_start"] + call["b_len"]])
        assert np.array_equal(part, C[k0:k1])


def pin_equal_element_case(orc) -> None:
    """merge_path.cu's tie case.  Expected values derived by hand from the
    definition: the walk takes A0 (1<=1), A1 (1<=1), B0 (2>1), A2 (2<=2),
    B1 (3>2), B2 (3>2), A3 (3<=4), then B3 because A is exhausted."""
    g = load_golden("equal_element_case.json")
    A, B = as_i32(g["A"]), as_i32(g["B"])
    assert list(orc.merge_i32(A, B)) == [1, 1, 1, 2, 2, 2, 3, 4]
    Av, Bv = tags(A.size, B.size)
    Ck, Cv = orc.merge_kv(A, Av, B, Bv)
    src = ["A%d" % v if v < U31 else "B%d" % (v - U31) for v in Cv]
    assert src == ["A0", "A1", "B0", "A2", "B1", "B2", "A3", "B3"], src
    assert list(Ck) == [1, 1, 1, 2, 2, 2, 3, 4]
    assert list(orc.co_rank_all(A, B)) == [0, 1, 2, 2, 3, 3, 3, 4, 4]


# ------------------------------------------------------ brute force / library

def _stable_sort_reference(A, B):
    """Brute force: stable sort by key of the tagged concatenation A||B."""
    keys = np.concatenate([A, B]).astype(np.int64)
    Av, Bv = tags(A.size, B.size)
    vals = np.concatenate([Av, Bv])
    order = np.argsort(keys, kind="stable")
    return keys[order].astype(np.int32), vals[order]


def _check_against_brute(orc, A, B) -> None:
    Av, Bv = tags(A.size, B.size)
    Ck, Cv = orc.merge_kv(A, Av, B, Bv)
    Rk, Rv = _stable_sort_reference(A, B)
    assert np.array_equal(Ck, Rk) and np.array_equal(Cv, Rv), (A, B)
    assert np.array_equal(orc.merge_i32(A, B), Rk), (A, B)
    # co-rank = number of A tags among the first k outputs
    I = orc.co_rank_all(A, B)
    from_a = np.concatenate([[0], np.cumsum(Rv < U31)])
    assert np.array_equal(I, from_a), (A, B)


def sorted_arrays(max_len: int, alphabet: int):
    for L in range(max_len + 1):
        for combo in itertools.combinations_with_replacement(range(alphabet), L):
            yield np.array(combo, dtype=np.int32)


def pin_exhaustive_tiny(orc, max_len: int = 5, alphabet: int = 3) -> None:
    """Every pair of sorted arrays of length <= max_len over {0..alphabet-1}."""
    arrs = list(sorted_arrays(max_len, alphabet))
    for A in arrs:
        for B in arrs:
            _check_against_brute(orc, A, B)


def _random_sorted(g, size, lo, hi):
    return np.sort(g.integers(lo, hi, size=size, dtype=np.int64)).astype(np.int32)


def pin_random_brute(orc, seed: int = 7, cases: int = 200) -> None:
    """Random sizes and value ranges, including the int32 extremes."""
    g = np.random.Generator(np.random.PCG64(seed))
    imin, imax = -(1 << 31), (1 << 31) - 1
    for c in range(cases):
        m, n = (int(x) for x in g.integers(0, 300, size=2))
        span = int(g.choice([2, 5, 50, 1 << 32]))
        if span == 1 << 32:
            A = _random_sorted(g, m, imin, imax + 1)
            B = _random_sorted(g, n, imin, imax + 1)
            # plant the extremes so the sign and the ends are exercised
            if m:
                A[0], A[-1] = imin, imax
            if n:
                B[0], B[-1] = imin, imax
            A.sort(); B.sort()
        else:
            base = int(g.integers(imin, imax - span))
            A = _random_sorted(g, m, base, base + span)
            B = _random_sorted(g, n, base, base + span)
        _check_against_brute(orc, A, B)


def pin_heapq_merge(orc, seed: int = 11, cases: int = 30) -> None:
    """heapq.merge is stable and takes the earlier iterable first on ties."""
    g = np.random.Generator(np.random.PCG64(seed))
    for c in range(cases):
        m, n = (int(x) for x in g.integers(0, 2000, size=2))
        A = _random_sorted(g, m, -20, 20)
        B = _random_sorted(g, n, -20, 20)
        Av, Bv = tags(m, n)
        ref = list(heapq.merge(zip(A.tolist(), Av.tolist()),
                               zip(B.tolist(), Bv.tolist()),
                               key=lambda p: p[0]))
        Ck, Cv = orc.merge_kv(A, Av, B, Bv)
        assert Ck.tolist() == [p[0] for p in ref]
        assert Cv.tolist() == [p[1] for p in ref]


def pin_rank_scatter(orc, seed: int = 13, cases: int = 20) -> None:
    """Each element's output position from its rank in the other array."""
    g = np.random.Generator(np.random.PCG64(seed))
    for c in range(cases):
        m, n = (int(x) for x in g.integers(0, 50000, size=2))
        span = int(g.choice([16, 1000, 1 << 31]))
        A = _random_sorted(g, m, -span, span)
        B = _random_sorted(g, n, -span, span)
        pos_a = np.arange(m) + np.searchsorted(B, A, side="left")
        pos_b = np.arange(n) + np.searchsorted(A, B, side="right")
        Rk = np.empty(m + n, dtype=np.int32)
        Rv = np.empty(m + n, dtype=np.uint32)
        Av, Bv = tags(m, n)
        Rk[pos_a], Rv[pos_a] = A, Av
        Rk[pos_b], Rv[pos_b] = B, Bv
        Ck, Cv = orc.merge_kv(A, Av, B, Bv)
        assert np.array_equal(Ck, Rk) and np.array_equal(Cv, Rv)
        # co-rank from the scatter: #A among the first k outputs
        I = orc.co_rank_all(A, B)
        marks = np.zeros(m + n, dtype=np.int64)
        marks[pos_a] = 1
        assert np.array_equal(I, np.concatenate([[0], np.cumsum(marks)]))


# ------------------------------------------------------------- closed forms

def pin_even_odd_closed_form(orc) -> None:
    """merge_path.cu's workload: A = 0,2,4,.. (m = 2^21+611), B = 1,3,5,..
    (n = 2^21).  Then C[k] = k for k < 2^22 and C[2^22 + r] = 2^22 + 2r for
    r < 611; co_rank(k) = ceil(k/2) for k <= 2^22 and k - 2^21 beyond."""
    m, n = (1 << 21) + 611, 1 << 21
    A = (2 * np.arange(m, dtype=np.int64)).astype(np.int32)
    B = (2 * np.arange(n, dtype=np.int64) + 1).astype(np.int32)
    C = orc.merge_i32(A, B)
    h = 1 << 22
    assert np.array_equal(C[:h], np.arange(h, dtype=np.int32))
    assert np.array_equal(C[h:], (h + 2 * np.arange(611)).astype(np.int32))
    I = orc.co_rank_all(A, B)
    k = np.arange(m + n + 1, dtype=np.int64)
    want = np.where(k <= h, (k + 1) // 2, k - (1 << 21))
    assert np.array_equal(I, want)


# --------------------------------------------------------------- invariants

def check_invariants(A, B, C, I) -> None:
    """i+j=k bounds, unit steps, acceptance test, order and permutation."""
    m, n = A.size, B.size
    k = np.arange(m + n + 1, dtype=np.int64)
    assert I.shape == (m + n + 1,)
    assert np.all(I >= np.maximum(0, k - n)) and np.all(I <= np.minimum(k, m))
    d = np.diff(I)
    assert np.all((d == 0) | (d == 1))
    J = k - I
    # acceptance test of the pages at every k: A[i-1] <= B[j] and B[j-1] < A[i]
    A64, B64 = A.astype(np.int64), B.astype(np.int64)
    lo_ok = (I == 0) | (J == n)
    ia, jb = np.clip(I - 1, 0, max(m - 1, 0)), np.clip(J, 0, max(n - 1, 0))
    if m and n:
        lo_ok |= A64[ia] <= B64[jb]
    hi_ok = (J == 0) | (I == m)
    ia2, jb2 = np.clip(I, 0, max(m - 1, 0)), np.clip(J - 1, 0, max(n - 1, 0))
    if m and n:
        hi_ok |= B64[jb2] < A64[ia2]
    assert np.all(lo_ok) and np.all(hi_ok)
    assert np.all(np.diff(C.astype(np.int64)) >= 0)
    # permutation: the same multiset of keys
    assert np.array_equal(np.sort(C), np.sort(np.concatenate([A, B])))
    # the step of I says where each output came from
    from_a = d == 1
    assert np.array_equal(C[from_a], A) and np.array_equal(C[~from_a], B)


def pin_invariants(orc, seed: int = 17, cases: int = 40) -> None:
    g = np.random.Generator(np.random.PCG64(seed))
    for c in range(cases):
        m, n = (int(x) for x in g.integers(0, 3000, size=2))
        span = int(g.choice([3, 100, 1 << 31]))
        A = _random_sorted(g, m, -span, span)
        B = _random_sorted(g, n, -span, span)
        check_invariants(A, B, orc.merge_i32(A, B), orc.co_rank_all(A, B))


def pin_kv_lexicographic(orc, m: int = 1 << 16, n: int = 1 << 16,
                         seed: int = 19) -> None:
    """With A payloads 0..m-1 and B payloads 2^31+0..n-1 ascending within each
    sorted array, the stable merge is strictly increasing in (key, payload),
    i.e. it equals a lexicographic sort of the concatenated pairs."""
    g = np.random.Generator(np.random.PCG64(seed))
    A = _random_sorted(g, m, 0, 256)
    B = _random_sorted(g, n, 0, 256)
    Av, Bv = tags(m, n)
    Ck, Cv = orc.merge_kv(A, Av, B, Bv)
    order = np.lexsort((np.concatenate([Av, Bv]), np.concatenate([A, B])))
    assert np.array_equal(Ck, np.concatenate([A, B])[order])
    assert np.array_equal(Cv, np.concatenate([Av, Bv])[order])


# --------------------------------------------- key types and descending order
#
# Float keys follow IEEE 754-2008 clause 5.10 (totalOrder).  The table below
# is written out by hand from that clause and the binary32 encoding (sign bit,
# 8 exponent bits, 23 fraction bits whose top bit marks a quiet NaN): every
# entry is a different datum, listed in increasing totalOrder.  The clause's
# rules used, in order: negative-sign NaNs lie below everything else and
# positive-sign NaNs above; -0 lies below +0; numbers otherwise by value; among
# NaNs of one sign, signaling lies nearer zero than quiet, and a larger payload
# lies farther from zero.

F32_TOTAL_ORDER = [
    (0xFFFFFFFF, "-qNaN, largest payload"),
    (0xFFC00001, "-qNaN, payload 1"),
    (0xFFC00000, "-qNaN, payload 0"),
    (0xFFBFFFFF, "-sNaN, largest payload"),
    (0xFF800001, "-sNaN, payload 1"),
    (0xFF800000, "-infinity"),
    (0xFF7FFFFF, "-largest finite (-3.4028235e38)"),
    (0xC0000000, "-2.0"),
    (0xBF800001, "-(1.0 + 2^-23)"),
    (0xBF800000, "-1.0"),
    (0x80800000, "-smallest normal (-2^-126)"),
    (0x807FFFFF, "-largest subnormal"),
    (0x80000001, "-smallest subnormal (-2^-149)"),
    (0x80000000, "-0.0"),
    (0x00000000, "+0.0"),
    (0x00000001, "+smallest subnormal (2^-149)"),
    (0x007FFFFF, "+largest subnormal"),
    (0x00800000, "+smallest normal (2^-126)"),
    (0x3F800000, "1.0"),
    (0x3F800001, "1.0 + 2^-23"),
    (0x40000000, "2.0"),
    (0x7F7FFFFF, "largest finite (3.4028235e38)"),
    (0x7F800000, "+infinity"),
    (0x7F800001, "+sNaN, payload 1"),
    (0x7FBFFFFF, "+sNaN, largest payload"),
    (0x7FC00000, "+qNaN, payload 0"),
    (0x7FC00001, "+qNaN, payload 1"),
    (0x7FFFFFFF, "+qNaN, largest payload"),
]


def f32_bits(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def pin_f32_total_order_table(orc) -> None:
    """The order relation on every pair of the hand-written table, both ways."""
    bits = [b for b, _ in F32_TOTAL_ORDER]
    vals = f32_bits(bits)
    for a in range(len(bits)):
        for b in range(len(bits)):
            assert orc.key_le(np.float32, vals[a], vals[b]) == (a <= b), \
                (F32_TOTAL_ORDER[a][1], F32_TOTAL_ORDER[b][1])
            assert orc.key_le(np.float32, vals[a], vals[b], descending=True) == (a >= b)


def _stable_by(rank, A, B):
    """Brute force: stable sort of the tagged concatenation A||B by rank(x)."""
    items = [(x, 0, i) for i, x in enumerate(A)] + [(x, 1, j) for j, x in enumerate(B)]
    order = sorted(range(len(items)), key=lambda t: rank(items[t][0]))
    return [items[t] for t in order]


def _check_typed(orc, A, B, rank, descending) -> None:
    want = _stable_by(rank, A, B)
    C = orc.merge_keys(A, B, descending)
    assert C.dtype == A.dtype
    assert np.array_equal(C.view(np.uint32),
                          np.array([w[0] for w in want], dtype=A.dtype).view(np.uint32))
    Av, Bv = tags(A.size, B.size)
    Ck, Cv = orc.merge_pairs(A, Av, B, Bv, descending)
    assert np.array_equal(Ck.view(np.uint32), C.view(np.uint32))
    want_tags = [(i if side == 0 else (1 << 31) + i) for _, side, i in want]
    assert np.array_equal(Cv, np.array(want_tags, dtype=np.uint32))


def pin_f32_special_brute(orc, seed: int = 37, cases: int = 300) -> None:
    """Random multisets over the table, sorted by table position (ascending)
    or its reverse (descending), against the brute-force stable sort."""
    g = np.random.Generator(np.random.PCG64(seed))
    bits = np.array([b for b, _ in F32_TOTAL_ORDER], dtype=np.uint32)
    for c in range(cases):
        m, n = (int(x) for x in g.integers(0, 12, size=2))
        desc = bool(c & 1)
        ia = np.sort(g.integers(0, len(bits), size=m))
        ib = np.sort(g.integers(0, len(bits), size=n))
        if desc:
            ia, ib = ia[::-1], ib[::-1]
        A, B = f32_bits(bits[ia]), f32_bits(bits[ib])
        pos = {int(b): r for r, b in enumerate(bits)}
        rank = (lambda x: -pos[int(np.float32(x).view(np.uint32))]) if desc else \
            (lambda x: pos[int(np.float32(x).view(np.uint32))])
        _check_typed(orc, A, B, rank, desc)


def pin_f32_numpy_finite(orc, seed: int = 41, cases: int = 40) -> None:
    """Finite keys, zeros of one sign only: the order is the ordinary numeric
    one, so numpy's stable sort of the concatenation is the merge (for
    descending, the stable sort of the negated keys)."""
    g = np.random.Generator(np.random.PCG64(seed))
    for c in range(cases):
        m, n = (int(x) for x in g.integers(0, 2000, size=2))
        desc = bool(c & 1)
        scale = float(g.choice([1.0, 1e-40, 1e30]))
        pool = (g.standard_normal(64) * scale).astype(np.float32)
        pool[pool == 0] = np.float32(0.0)
        A = np.sort(g.choice(pool, size=m)).astype(np.float32)
        B = np.sort(g.choice(pool, size=n)).astype(np.float32)
        if desc:
            A, B = A[::-1].copy(), B[::-1].copy()
        cat = np.concatenate([A, B])
        order = np.argsort(-cat if desc else cat, kind="stable")
        assert np.array_equal(orc.merge_keys(A, B, desc), cat[order])


def pin_integer_kinds_brute(orc, seed: int = 43, cases: int = 200) -> None:
    """int32 and uint32 keys, both orders, including the type extremes, against
    the brute-force stable sort by Python integer value."""
    g = np.random.Generator(np.random.PCG64(seed))
    for c in range(cases):
        dtype = np.uint32 if c % 4 < 2 else np.int32
        desc = bool(c & 1)
        info = np.iinfo(dtype)
        pool = np.array([info.min, info.min + 1, -1 if dtype == np.int32 else 1 << 31,
                         0, 1, (1 << 31) - 1, info.max - 1, info.max], dtype=np.int64)
        pool = np.concatenate([pool, g.integers(info.min, int(info.max) + 1, size=4)])
        m, n = (int(x) for x in g.integers(0, 14, size=2))
        A = np.sort(g.choice(pool, size=m)).astype(dtype)
        B = np.sort(g.choice(pool, size=n)).astype(dtype)
        if desc:
            A, B = A[::-1].copy(), B[::-1].copy()
        rank = (lambda x: -int(x)) if desc else (lambda x: int(x))
        _check_typed(orc, A, B, rank, desc)


def pin_integer_kinds_numpy(orc, seed: int = 47, cases: int = 24) -> None:
    """Larger int32 / uint32 cases against numpy's stable argsort (descending:
    of the reversed keys, max - x, computed in int64)."""
    g = np.random.Generator(np.random.PCG64(seed))
    for c in range(cases):
        dtype = np.uint32 if c % 4 < 2 else np.int32
        desc = bool(c & 1)
        info = np.iinfo(dtype)
        span = int(g.choice([4, 1 << 32]))
        lo = int(info.min) if span > 4 else 0
        m, n = (int(x) for x in g.integers(0, 5000, size=2))
        A = np.sort(g.integers(lo, lo + span, size=m)).astype(dtype)
        B = np.sort(g.integers(lo, lo + span, size=n)).astype(dtype)
        if desc:
            A, B = A[::-1].copy(), B[::-1].copy()
        cat = np.concatenate([A, B])
        key = int(info.max) - cat.astype(np.int64) if desc else cat.astype(np.int64)
        order = np.argsort(key, kind="stable")
        assert np.array_equal(orc.merge_keys(A, B, desc), cat[order])


def pin_typed_i32_worked_example(orc) -> None:
    """The typed routine on int32 ascending reproduces the page's worked
    example output (12-merge/02), and reversing both inputs and the order
    gives the reversed output up to the tie rule (checked through tags)."""
    g = load_golden("worked_example_corank.json")
    A, B = as_i32(g["A"]), as_i32(g["B"])
    assert np.array_equal(orc.merge_keys(A, B), orc.merge_i32(A, B))
    assert orc.merge_keys(A, B).tolist() == [1, 7, 7, 8, 9, 10, 10, 10, 12]
    Ck = orc.merge_keys(A[::-1].copy(), B[::-1].copy(), descending=True)
    assert Ck.tolist() == [12, 10, 10, 10, 9, 8, 7, 7, 1]


# binary64 (sign bit, 11 exponent bits, 52 fraction bits whose top bit marks
# a quiet NaN), in increasing totalOrder by the same rules, written out by
# hand.
F64_TOTAL_ORDER = [
    (0xFFFFFFFFFFFFFFFF, "-qNaN, largest payload"),
    (0xFFF8000000000001, "-qNaN, payload 1"),
    (0xFFF8000000000000, "-qNaN, payload 0"),
    (0xFFF7FFFFFFFFFFFF, "-sNaN, largest payload"),
    (0xFFF0000000000001, "-sNaN, payload 1"),
    (0xFFF0000000000000, "-infinity"),
    (0xFFEFFFFFFFFFFFFF, "-largest finite"),
    (0xC000000000000000, "-2.0"),
    (0xBFF0000000000001, "-(1.0 + 2^-52)"),
    (0xBFF0000000000000, "-1.0"),
    (0xBFEFFFFFFFFFFFFF, "-(1.0 - 2^-53)"),
    (0x8010000000000000, "-smallest normal (-2^-1022)"),
    (0x800FFFFFFFFFFFFF, "-largest subnormal"),
    (0x8000000000000001, "-smallest subnormal (-2^-1074)"),
    (0x8000000000000000, "-0.0"),
    (0x0000000000000000, "+0.0"),
    (0x0000000000000001, "+smallest subnormal (2^-1074)"),
    (0x000FFFFFFFFFFFFF, "+largest subnormal"),
    (0x0010000000000000, "+smallest normal (2^-1022)"),
    (0x3FEFFFFFFFFFFFFF, "1.0 - 2^-53"),
    (0x3FF0000000000000, "1.0"),
    (0x3FF0000000000001, "1.0 + 2^-52"),
    (0x4000000000000000, "2.0"),
    (0x7FEFFFFFFFFFFFFF, "largest finite"),
    (0x7FF0000000000000, "+infinity"),
    (0x7FF0000000000001, "+sNaN, payload 1"),
    (0x7FF7FFFFFFFFFFFF, "+sNaN, largest payload"),
    (0x7FF8000000000000, "+qNaN, payload 0"),
    (0x7FF8000000000001, "+qNaN, payload 1"),
    (0x7FFFFFFFFFFFFFFF, "+qNaN, largest payload"),
]


def f64_bits(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint64).view(np.float64)


def tags64(m: int, n: int):
    """64-bit payload tags: A element i -> i, B element j -> 2^63 + j."""
    return (np.arange(m, dtype=np.uint64),
            (np.uint64(1 << 63) + np.arange(n, dtype=np.uint64)).astype(np.uint64))


def pin_f64_total_order_table(orc) -> None:
    bits = [b for b, _ in F64_TOTAL_ORDER]
    vals = f64_bits(bits)
    for a in range(len(bits)):
        for b in range(len(bits)):
            assert orc.key_le(np.float64, vals[a], vals[b]) == (a <= b), \
                (F64_TOTAL_ORDER[a][1], F64_TOTAL_ORDER[b][1])
            assert orc.key_le(np.float64, vals[a], vals[b], descending=True) == (a >= b)


def _check_typed64(orc, A, B, rank, descending) -> None:
    """As _check_typed, with 64-bit payload tags as well as 32-bit ones."""
    _check_typed(orc, A, B, rank, descending)
    want = _stable_by(rank, A, B)
    Av, Bv = tags64(A.size, B.size)
    Ck, Cv = orc.merge_pairs(A, Av, B, Bv, descending)
    assert Cv.dtype == np.uint64
    want_tags = [(i if side == 0 else (1 << 63) + i) for _, side, i in want]
    assert np.array_equal(Cv, np.array(want_tags, dtype=np.uint64))
    assert np.array_equal(Ck.view(np.uint8), orc.merge_keys(A, B, descending).view(np.uint8))


def pin_f64_special_brute(orc, seed: int = 53, cases: int = 200) -> None:
    g = np.random.Generator(np.random.PCG64(seed))
    bits = np.array([b for b, _ in F64_TOTAL_ORDER], dtype=np.uint64)
    pos = {int(b): r for r, b in enumerate(bits)}
    for c in range(cases):
        m, n = (int(x) for x in g.integers(0, 12, size=2))
        desc = bool(c & 1)
        ia = np.sort(g.integers(0, len(bits), size=m))
        ib = np.sort(g.integers(0, len(bits), size=n))
        if desc:
            ia, ib = ia[::-1], ib[::-1]
        A, B = f64_bits(bits[ia]), f64_bits(bits[ib])
        key = lambda x: pos[int(np.float64(x).view(np.uint64))]
        rank = (lambda x: -key(x)) if desc else key
        _check_typed64(orc, A, B, rank, desc)


def pin_f64_numpy_finite(orc, seed: int = 59, cases: int = 30) -> None:
    """Finite binary64 keys, zeros of one sign only, against numpy's stable
    sort (descending: of the negated keys)."""
    g = np.random.Generator(np.random.PCG64(seed))
    for c in range(cases):
        m, n = (int(x) for x in g.integers(0, 2000, size=2))
        desc = bool(c & 1)
        scale = float(g.choice([1.0, 1e-300, 1e300]))
        pool = g.standard_normal(64) * scale
        pool[pool == 0] = 0.0
        A = np.sort(g.choice(pool, size=m))
        B = np.sort(g.choice(pool, size=n))
        if desc:
            A, B = A[::-1].copy(), B[::-1].copy()
        cat = np.concatenate([A, B])
        order = np.argsort(-cat if desc else cat, kind="stable")
        assert np.array_equal(orc.merge_keys(A, B, desc), cat[order])


def pin_integer64_kinds_brute(orc, seed: int = 61, cases: int = 200) -> None:
    """int64 and uint64 keys, both orders, including the type extremes and
    keys that differ only in their high or only in their low 32 bits."""
    g = np.random.Generator(np.random.PCG64(seed))
    for c in range(cases):
        dtype = np.uint64 if c % 4 < 2 else np.int64
        desc = bool(c & 1)
        info = np.iinfo(dtype)
        lo, hi = int(info.min), int(info.max)
        pool = [lo, lo + 1, 0, 1, (1 << 32) - 1, 1 << 32, (1 << 32) + 1, hi - 1, hi,
                (1 << 31) - 1, 1 << 31]
        if dtype == np.int64:
            pool += [-1, -(1 << 32), -(1 << 32) + 1, -(1 << 31)]
        else:
            pool += [1 << 63, (1 << 63) + 1, (1 << 63) - 1]
        pool += [int(x) for x in g.integers(lo, hi, size=4, dtype=dtype, endpoint=True)]
        pool = sorted(set(pool))
        m, n = (int(x) for x in g.integers(0, 14, size=2))
        A = np.array(sorted(int(pool[i]) for i in g.integers(0, len(pool), size=m)),
                     dtype=dtype)
        B = np.array(sorted(int(pool[i]) for i in g.integers(0, len(pool), size=n)),
                     dtype=dtype)
        if desc:
            A, B = A[::-1].copy(), B[::-1].copy()
        rank = (lambda x: -int(x)) if desc else (lambda x: int(x))
        _check_typed64(orc, A, B, rank, desc)


def pin_integer64_kinds_sorted(orc, seed: int = 67, cases: int = 16) -> None:
    """Larger int64 / uint64 cases against Python's stable sort of the
    concatenation by integer value (descending: by its negation)."""
    g = np.random.Generator(np.random.PCG64(seed))
    for c in range(cases):
        dtype = np.uint64 if c % 4 < 2 else np.int64
        desc = bool(c & 1)
        info = np.iinfo(dtype)
        m, n = (int(x) for x in g.integers(0, 3000, size=2))
        if c % 8 < 4:
            draw = lambda k: g.integers(info.min, info.max, size=k, dtype=dtype, endpoint=True)
        else:
            base = int(g.integers(0, 1 << 20)) << 32
            draw = lambda k: (np.uint64(base) + g.integers(0, 8, size=k).astype(np.uint64)
                              ).astype(dtype)
        A, B = np.sort(draw(m)), np.sort(draw(n))
        if desc:
            A, B = A[::-1].copy(), B[::-1].copy()
        cat = [int(x) for x in np.concatenate([A, B])]
        order = sorted(range(len(cat)), key=(lambda t: -cat[t]) if desc else (lambda t: cat[t]))
        want = np.array([cat[t] for t in order], dtype=dtype)
        assert np.array_equal(orc.merge_keys(A, B, desc), want)


# ---------------------------------------------- batched merges and the sort


def _rank_of(dtype, descending):
    """Python rank key of one key value, for brute force: integers by value,
    floats by position in the hand-written totalOrder tables (only table
    values are drawn), reversed for descending."""
    if np.dtype(dtype).kind == "f":
        table = F32_TOTAL_ORDER if np.dtype(dtype) == np.float32 else F64_TOTAL_ORDER
        bits = np.uint32 if np.dtype(dtype) == np.float32 else np.uint64
        pos = {b: r for r, (b, _) in enumerate(table)}
        key = lambda x: pos[int(np.asarray(x, dtype=dtype).view(bits))]
    else:
        key = lambda x: int(x)
    return (lambda x: -key(x)) if descending else key


def _draw_keys(g, dtype, size):
    if np.dtype(dtype).kind == "f":
        table = F32_TOTAL_ORDER if np.dtype(dtype) == np.float32 else F64_TOTAL_ORDER
        bits = np.uint32 if np.dtype(dtype) == np.float32 else np.uint64
        pick = np.array([b for b, _ in table], dtype=bits)
        return pick[g.integers(0, len(pick), size=size)].view(dtype)
    info = np.iinfo(dtype)
    pool = np.array([info.min, info.min + 1, 0, 1, info.max - 1, info.max], dtype=dtype)
    mixed = np.concatenate([pool, g.integers(info.min, info.max, size=4, dtype=dtype,
                                             endpoint=True)])
    return mixed[g.integers(0, mixed.size, size=size)]


def pin_sort_brute(orc, seed: int = 71, cases: int = 240) -> None:
    """Stable sort against Python's stable sorted() of (rank, input index),
    every key type, both orders, with 4- and 8-byte payload tags."""
    g = np.random.Generator(np.random.PCG64(seed))
    dtypes = [np.int32, np.uint32, np.float32, np.int64, np.uint64, np.float64]
    for c in range(cases):
        dtype = dtypes[c % len(dtypes)]
        desc = bool((c // len(dtypes)) & 1)
        n = int(g.integers(0, 40))
        K = _draw_keys(g, dtype, n)
        rank = _rank_of(dtype, desc)
        order = sorted(range(n), key=lambda t: rank(K[t]))
        got = orc.sort(K, descending=desc)
        assert np.array_equal(got.view(np.uint8), K[order].view(np.uint8))
        for vdt in (np.uint32, np.uint64):
            V = np.arange(n, dtype=vdt) + vdt(7)
            gk, gv = orc.sort(K, V, descending=desc)
            assert np.array_equal(gv, V[order])
            assert np.array_equal(gk.view(np.uint8), K[order].view(np.uint8))


def pin_sort_numpy(orc, seed: int = 73, cases: int = 12) -> None:
    """Larger sorts against numpy's stable argsort (descending: of the
    negated keys, in int64 for integers, for finite floats as is)."""
    g = np.random.Generator(np.random.PCG64(seed))
    for c in range(cases):
        dtype = [np.int32, np.float32, np.int64, np.float64][c % 4]
        desc = bool(c & 4)
        n = int(g.integers(1, 30000))
        if np.dtype(dtype).kind == "f":
            K = (g.standard_normal(n) * 100).round(1).astype(dtype)
            K[K == 0] = 0.0
            key = -K if desc else K
        else:
            K = g.integers(-50, 50, size=n).astype(dtype)
            key = -K.astype(np.int64) if desc else K
        idx = np.argsort(key, kind="stable")
        V = np.arange(n, dtype=np.uint32)
        gk, gv = orc.sort(K, V, descending=desc)
        assert np.array_equal(gk, K[idx]) and np.array_equal(gv, V[idx])


def pin_sort_permutation_of_tiny(orc) -> None:
    """Every arrangement of a small multiset sorts to the same keys, and the
    payloads of equal keys keep their input order (exhaustive, n <= 6)."""
    import itertools
    for keys in ([3, 1, 2, 1, 3, 1], [5, 5, 5, 5], [2, 1, 0, -1, -2, 7]):
        want = sorted(keys)
        for perm in set(itertools.permutations(keys)):
            K = np.array(perm, dtype=np.int32)
            V = np.arange(len(perm), dtype=np.uint32)
            gk, gv = orc.sort(K, V)
            assert gk.tolist() == want
            for a, b in zip(range(len(perm)), range(1, len(perm))):
                if gk[a] == gk[b]:
                    assert gv[a] < gv[b]


def pin_batched_against_pairs(orc, seed: int = 79, cases: int = 60) -> None:
    """A batch of merges equals, merge by merge, numpy's stable sort of that
    merge's A||B (ties: A first, then input order), placed one after
    another; empty merges and empty sides included."""
    g = np.random.Generator(np.random.PCG64(seed))
    for c in range(cases):
        pairs = int(g.integers(1, 12))
        desc = bool(c & 1)
        la = g.integers(0, 30, size=pairs) * (g.random(pairs) > 0.2)
        lb = g.integers(0, 30, size=pairs) * (g.random(pairs) > 0.2)
        a_off = np.concatenate([[0], np.cumsum(la)]).astype(np.int64)
        b_off = np.concatenate([[0], np.cumsum(lb)]).astype(np.int64)
        A = np.empty(int(a_off[-1]), dtype=np.int32)
        B = np.empty(int(b_off[-1]), dtype=np.int32)
        want = []
        want_tags = []
        for p in range(pairs):
            a = np.sort(g.integers(-5, 5, size=int(la[p]))).astype(np.int32)
            b = np.sort(g.integers(-5, 5, size=int(lb[p]))).astype(np.int32)
            if desc:
                a, b = a[::-1].copy(), b[::-1].copy()
            A[a_off[p]:a_off[p + 1]] = a
            B[b_off[p]:b_off[p + 1]] = b
            cat = np.concatenate([a, b])
            tag = np.concatenate([a_off[p] + np.arange(a.size), (1 << 31) + b_off[p] +
                                  np.arange(b.size)])
            idx = np.argsort(-cat.astype(np.int64) if desc else cat, kind="stable")
            want.append(cat[idx])
            want_tags.append(tag[idx])
        Av = np.arange(A.size, dtype=np.uint32)
        Bv = (U31 + np.arange(B.size, dtype=np.uint32)).astype(np.uint32)
        Ck, Cv = orc.merge_batched(A, a_off, B, b_off, Av, Bv, descending=desc)
        assert np.array_equal(Ck, np.concatenate(want))
        assert np.array_equal(Cv, np.concatenate(want_tags).astype(np.uint32))
        assert np.array_equal(orc.merge_batched(A, a_off, B, b_off, descending=desc), Ck)


def _sorted_runs(g, dtype, n, run, desc):
    """Keys of dtype whose consecutive runs of ``run`` are each sorted in the
    key order (rank), with many ties across runs."""
    rank = _rank_of(dtype, desc)
    K = _draw_keys(g, dtype, n)
    if n and g.random() < 0.5:
        K = K[g.integers(0, max(1, min(n, 4)), size=n)]  # few distinct keys
    for s in range(0, n, run):
        part = K[s:s + run]
        K[s:s + run] = part[sorted(range(part.size), key=lambda t: rank(part[t]))]
    return K


def pin_merge_runs_brute(orc, seed: int = 83, cases: int = 240) -> None:
    """A k-way pass equals, group by group, Python's stable sorted() of
    (rank, input index) over that group of runs: the stable merge, ties to
    the earlier run and within a run to the earlier element.  Every key type,
    both orders, 4- and 8-byte payload tags, ragged last group and run."""
    g = np.random.Generator(np.random.PCG64(seed))
    dtypes = [np.int32, np.uint32, np.float32, np.int64, np.uint64, np.float64]
    for c in range(cases):
        dtype = dtypes[c % len(dtypes)]
        desc = bool((c // len(dtypes)) & 1)
        n = int(g.integers(0, 60))
        run = int(g.integers(1, 9))
        ways = int(g.integers(1, 9)) if c % 5 else int(g.integers(9, 65))
        K = _sorted_runs(g, dtype, n, run, desc)
        rank = _rank_of(dtype, desc)
        order = []
        for g0 in range(0, n, run * ways):
            grp = range(g0, min(n, g0 + run * ways))
            order += sorted(grp, key=lambda t: rank(K[t]))
        got = orc.merge_runs(K, run, ways, descending=desc)
        assert np.array_equal(got.view(np.uint8), K[order].view(np.uint8))
        for vdt in (np.uint32, np.uint64):
            V = np.arange(n, dtype=vdt) + vdt(5)
            gk, gv = orc.merge_runs(K, run, ways, V, descending=desc)
            assert np.array_equal(gv, V[order])
            assert np.array_equal(gk.view(np.uint8), K[order].view(np.uint8))


def pin_merge_runs_two_way_is_batched(orc, seed: int = 89, cases: int = 40) -> None:
    """With two ways, a pass is the batch of 2-way merges of adjacent runs
    (left run as A): the co-rank merge the pages define, merge by merge."""
    g = np.random.Generator(np.random.PCG64(seed))
    for c in range(cases):
        desc = bool(c & 1)
        n = int(g.integers(1, 400))
        run = int(g.integers(1, 40))
        K = _sorted_runs(g, np.int32, n, run, desc)
        V = np.arange(n, dtype=np.uint32)
        starts = np.arange(0, n, 2 * run, dtype=np.int64)
        a_end = np.minimum(starts + run, n)
        b_end = np.minimum(starts + 2 * run, n)
        a_idx = np.concatenate([np.arange(s, e) for s, e in zip(starts, a_end)])
        b_idx = np.concatenate([np.arange(s, e) for s, e in zip(a_end, b_end)] +
                               [np.zeros(0, dtype=np.int64)])
        a_off = np.concatenate([[0], np.cumsum(a_end - starts)]).astype(np.int64)
        b_off = np.concatenate([[0], np.cumsum(b_end - a_end)]).astype(np.int64)
        wk, wv = orc.merge_batched(K[a_idx], a_off, K[b_idx], b_off, V[a_idx],
                                   V[b_idx].astype(np.uint32), descending=desc)
        gk, gv = orc.merge_runs(K, run, 2, V, descending=desc)
        assert np.array_equal(gk, wk) and np.array_equal(gv, wv)


def pin_merge_runs_composes(orc, seed: int = 97, cases: int = 40) -> None:
    """Stable merges compose: one 4-way pass over runs of r equals a 2-way
    pass over runs of r and then one over runs of 2r; 8 ways equal 2 x 4 and
    4 x 2.  Repeated passes from runs of one element give the stable sort."""
    g = np.random.Generator(np.random.PCG64(seed))
    for c in range(cases):
        dtype = [np.int32, np.float64][c & 1]
        desc = bool(c & 2)
        n = int(g.integers(1, 500))
        run = int(g.integers(1, 20))
        K = _sorted_runs(g, dtype, n, run, desc)
        V = np.arange(n, dtype=np.uint32)
        k2, v2 = orc.merge_runs(K, run, 2, V, descending=desc)
        k22, v22 = orc.merge_runs(k2, 2 * run, 2, v2, descending=desc)
        k4, v4 = orc.merge_runs(K, run, 4, V, descending=desc)
        assert np.array_equal(v4, v22) and np.array_equal(k4.view(np.uint8), k22.view(np.uint8))
        k24, v24 = orc.merge_runs(k2, 2 * run, 4, v2, descending=desc)
        k42, v42 = orc.merge_runs(k4, 4 * run, 2, v4, descending=desc)
        k8, v8 = orc.merge_runs(K, run, 8, V, descending=desc)
        assert np.array_equal(v8, v24) and np.array_equal(v8, v42)
        # a full sort by passes of 3 ways from runs of one element
        U = _draw_keys(g, dtype, n)
        k, v, r = U, V, 1
        while r < n:
            k, v = orc.merge_runs(k, r, 3, v, descending=desc)
            r *= 3
        sk, sv = orc.sort(U, V, descending=desc)
        assert np.array_equal(v, sv) and np.array_equal(k.view(np.uint8), sk.view(np.uint8))


def pin_merge_runs_special(orc) -> None:
    """Closed cases: all keys equal leave every element in place; runs that
    are already in order across their boundaries pass through; runs whose key
    ranges fall from run to run come out last run first; one way, or a run covering the
    whole input, is the identity."""
    n = 37
    V = np.arange(n, dtype=np.uint32)
    same = np.full(n, 4, dtype=np.int32)
    for run, ways in ((1, 2), (3, 4), (5, 7), (1, 64), (36, 2)):
        k, v = orc.merge_runs(same, run, ways, V)
        assert np.array_equal(v, V)
    inc = np.arange(n, dtype=np.int32)
    for run, ways in ((1, 2), (4, 3), (10, 4)):
        k, v = orc.merge_runs(inc, run, ways, V)
        assert np.array_equal(v, V)
    # 4 runs of 3, each run's keys above the next run's: the group comes out
    # as run 3, run 2, run 1, run 0
    K = np.array([9, 10, 11, 6, 7, 8, 3, 4, 5, 0, 1, 2], dtype=np.int32)
    k, v = orc.merge_runs(K, 3, 4, np.arange(12, dtype=np.uint32))
    assert k.tolist() == list(range(12))
    assert v.tolist() == [9, 10, 11, 6, 7, 8, 3, 4, 5, 0, 1, 2]
    # reversed, each run descends and the largest keys sit in the last run:
    # in descending order the group again comes out last run first
    kd, vd = orc.merge_runs(K[::-1].copy(), 3, 4, np.arange(12, dtype=np.uint32),
                            descending=True)
    assert kd.tolist() == list(range(11, -1, -1))
    assert vd.tolist() == [9, 10, 11, 6, 7, 8, 3, 4, 5, 0, 1, 2]
    R = np.array([5, 1, 4, 2, 3], dtype=np.int32)
    assert orc.merge_runs(R, 1, 1).tolist() == R.tolist()
    srt = np.array([1, 3, 5, 2, 4], dtype=np.int32)
    assert orc.merge_runs(srt, 5, 2).tolist() == srt.tolist()
    assert orc.merge_runs(np.zeros(0, dtype=np.int32), 4, 4).size == 0


ALL_PINS = [
    pin_worked_example,
    pin_equal_element_case,
    pin_exhaustive_tiny,
    pin_random_brute,
    pin_heapq_merge,
    pin_rank_scatter,
    pin_even_odd_closed_form,
    pin_invariants,
    pin_kv_lexicographic,
    pin_f32_total_order_table,
    pin_f32_special_brute,
    pin_f32_numpy_finite,
    pin_integer_kinds_brute,
    pin_integer_kinds_numpy,
    pin_typed_i32_worked_example,
    pin_f64_total_order_table,
    pin_f64_special_brute,
    pin_f64_numpy_finite,
    pin_integer64_kinds_brute,
    pin_integer64_kinds_sorted,
    pin_sort_brute,
    pin_sort_numpy,
    pin_sort_permutation_of_tiny,
    pin_batched_against_pairs,
    pin_merge_runs_brute,
    pin_merge_runs_two_way_is_batched,
    pin_merge_runs_composes,
    pin_merge_runs_special,
]


def run_all(orc) -> list:
    """Run every pin; return the names of the pins that failed."""
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    return failed

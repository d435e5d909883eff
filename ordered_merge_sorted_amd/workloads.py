"""Seeded synthetic inputs for the merge: the five workloads and small random cases.

This module holds no merge arithmetic.  It only draws random numbers and sorts
each input array on its own; both the CPU oracle (in the tests) and the HIP
path consume the arrays it returns.

Sorted iid-uniform arrays are drawn bucket by bucket: the value range is cut
into ``nb`` equal buckets, the bucket counts are one multinomial draw, and each
bucket's values are drawn iid uniform inside the bucket and sorted.  The result
has exactly the distribution of "draw N values iid uniform over the range, then
sort ascending", but the buckets are independent, so they are drawn and sorted
in parallel threads (numpy releases the GIL in both).  Every bucket has its own
child generator spawned from the workload's seed, so the output does not depend
on the thread count.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Callable, Dict, Tuple

import numpy as np

SEED_BASE = 20261200


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def sorted_uniform(seed, count: int, lo: int, hi: int, nb: int = 256) -> np.ndarray:
    """``count`` int32 values iid uniform over [lo, hi), sorted ascending.

    ``hi - lo`` must be divisible by the bucket count (all ranges used here are
    powers of two).  ``seed`` is an int or a ``numpy.random.SeedSequence``.
    """
    span = hi - lo
    if span <= 0:
        raise ValueError("empty range")
    nb = min(nb, span)
    if span % nb:
        raise ValueError("range %d not divisible into %d buckets" % (span, nb))
    width = span // nb
    ss = seed if isinstance(seed, np.random.SeedSequence) else np.random.SeedSequence(seed)
    top, *children = ss.spawn(nb + 1)
    counts = np.random.Generator(np.random.PCG64(top)).multinomial(
        count, np.full(nb, 1.0 / nb))
    offsets = np.zeros(nb + 1, dtype=np.int64)
    np.cumsum(counts, out=offsets[1:])
    out = np.empty(count, dtype=np.int32)

    def fill(b: int) -> None:
        c = int(counts[b])
        if c == 0:
            return
        g = np.random.Generator(np.random.PCG64(children[b]))
        base = lo + b * width
        v = g.integers(0, width, size=c, dtype=np.int64) + base
        v.sort()
        out[offsets[b]:offsets[b + 1]] = v.astype(np.int32)

    if count >= (1 << 20):
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nb)))
    else:
        for b in range(nb):
            fill(b)
    return out


@dataclass(frozen=True)
class Workload:
    """One synthetic merge workload.  ``make()`` returns (A, B) for key-only
    workloads and (A_keys, A_vals, B_keys, B_vals) for key+payload ones."""
    name: str
    m: int
    n: int
    kv: bool
    seed: int
    description: str
    make: Callable[[], Tuple[np.ndarray, ...]]

    @property
    def total(self) -> int:
        return self.m + self.n

    @property
    def bytes_per_element(self) -> int:
        return 8 if self.kv else 4

    @property
    def roofline_bytes(self) -> int:
        """Bytes the merge cannot avoid: every element read once, written once."""
        return 2 * self.total * self.bytes_per_element


def _pair(seed: int, m: int, lo_a: int, hi_a: int, n: int, lo_b: int, hi_b: int):
    sa, sb = np.random.SeedSequence(seed).spawn(2)
    return sorted_uniform(sa, m, lo_a, hi_a), sorted_uniform(sb, n, lo_b, hi_b)


def _ties_4096():
    return _pair(SEED_BASE + 1, 65563, 0, 4096, 65536, 0, 4096)


def _even_odd():
    m, n = (1 << 21) + 611, 1 << 21
    A = (2 * np.arange(m, dtype=np.int64)).astype(np.int32)
    B = (2 * np.arange(n, dtype=np.int64) + 1).astype(np.int32)
    return A, B


def _uniform_2p28():
    return _pair(SEED_BASE + 3, 1 << 28, -(1 << 31), 1 << 31,
                 1 << 28, -(1 << 31), 1 << 31)


def _kv_ties_256():
    m = n = 1 << 26
    Ak, Bk = _pair(SEED_BASE + 4, m, 0, 256, n, 0, 256)
    Av = np.arange(m, dtype=np.uint32)
    Bv = (np.uint32(1 << 31) + np.arange(n, dtype=np.uint32)).astype(np.uint32)
    return Ak, Av, Bk, Bv


def _skewed():
    return _pair(SEED_BASE + 5, 1 << 27, 0, 1 << 30,
                 1 << 24, 1 << 29, (1 << 29) + (1 << 20))


WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    Workload("ties_4096_65563x65536", 65563, 65536, False, SEED_BASE + 1,
             "int32 keys iid uniform in [0,4096), m=65,563, n=65,536, sorted; "
             "heavy cross-array ties", _ties_4096),
    Workload("even_odd_2p21", (1 << 21) + 611, 1 << 21, False, 0,
             "A = 0,2,4,... (m=2^21+611), B = 1,3,5,... (n=2^21); all distinct, "
             "odd total, last 611 outputs from A alone", _even_odd),
    Workload("uniform_i32_2p28x2p28", 1 << 28, 1 << 28, False, SEED_BASE + 3,
             "int32 keys iid uniform over the full int32 range, m=n=2^28, sorted; "
             "2 GiB in, 2 GiB out", _uniform_2p28),
    Workload("kv_ties_256_2p26x2p26", 1 << 26, 1 << 26, True, SEED_BASE + 4,
             "int32 keys iid uniform in [0,256) sorted, uint32 payload = sorted "
             "position (A: 0..m-1, B: 2^31+0..n-1), m=n=2^26", _kv_ties_256),
    Workload("skewed_2p27x2p24", 1 << 27, 1 << 24, False, SEED_BASE + 5,
             "A: 2^27 keys iid uniform in [0,2^30); B: 2^24 keys iid uniform in "
             "[2^29, 2^29+2^20); both sorted", _skewed),
]}

# Workload order used by tests and the benchmark (smallest first).
ORDER = list(WORKLOADS)

HEADLINE = "uniform_i32_2p28x2p28"


def random_case(seed: int, m: int, n: int, lo: int = -50, hi: int = 50,
                kv: bool = False):
    """Small random sorted case with many ties.  Payloads (kv) are distinct:
    A gets 0..m-1 and B gets 2^31 + 0..n-1."""
    g = np.random.Generator(np.random.PCG64(seed))
    A = np.sort(g.integers(lo, hi, size=m, dtype=np.int64)).astype(np.int32)
    B = np.sort(g.integers(lo, hi, size=n, dtype=np.int64)).astype(np.int32)
    if not kv:
        return A, B
    Av = np.arange(m, dtype=np.uint32)
    Bv = (np.uint32(1 << 31) + np.arange(n, dtype=np.uint32)).astype(np.uint32)
    return A, Av, B, Bv

"""Host model of the co-rank binary search, as the pages describe it.

This is neither the oracle nor the HIP path; it models the search the device
code runs, so that its properties can be checked on the CPU: the printed trace
of co_rank(3) on the worked example, termination (the half-step must round
up), and the bound on the number of steps.

The search (page 'Co-rank Function ... and Basic Parallel Merge Kernel',
section 'Binary-Search Implementation' and the formula table; page
'merge_path.cu', the co-rank routine and its comment): keep a candidate split
(i, j) with i + j = k, starting from the upper bound i = min(k, m), with lower
bounds i_low = max(0, k - n) and j_low = max(0, k - m).  If A[i-1] > B[j] the
split holds too many A elements: move i down (and j up) by half the distance
to i_low, rounded up, and raise j_low to the old j.  Otherwise, if
B[j-1] >= A[i] it holds too many B elements: move j down (and i up) by half
the distance to j_low, rounded up, and raise i_low to the old i.  Otherwise the
split is accepted.  The '>' against '>=' asymmetry puts equal A keys first.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence


@dataclass
class SearchResult:
    i: int
    steps: int                      # adjustments made before acceptance
    trace: List[dict] = field(default_factory=list)
    finished: bool = True           # False when the step cap stopped it


def _half_up(d: int) -> int:
    return (d + 1) >> 1


def _half_down(d: int) -> int:
    return d >> 1


def co_rank_search(k: int, A: Sequence[int], B: Sequence[int],
                   round_up: bool = True, max_steps: Optional[int] = None,
                   record: bool = False) -> SearchResult:
    m, n = len(A), len(B)
    half = _half_up if round_up else _half_down
    i = min(k, m)
    j = k - i
    i_low = max(0, k - n)
    j_low = max(0, k - m)
    res = SearchResult(i=-1, steps=0)
    while True:
        too_many_a = i > 0 and j < n and A[i - 1] > B[j]
        too_many_b = (not too_many_a) and j > 0 and i < m and B[j - 1] >= A[i]
        row = {"iter": res.steps, "i_low": i_low, "i": i, "j": j, "j_low": j_low}
        if too_many_a:
            d = half(i - i_low)
            row.update(verdict="i too large", delta=d)
            j_low = j
            i, j = i - d, j + d
        elif too_many_b:
            d = half(j - j_low)
            row.update(verdict="j too large", delta=d)
            i_low = i
            i, j = i + d, j - d
        else:
            row.update(verdict="accept", delta=None)
            if record:
                res.trace.append(row)
            res.i = i
            return res
        if record:
            res.trace.append(row)
        res.steps += 1
        if max_steps is not None and res.steps >= max_steps:
            res.finished = False
            res.i = i
            return res


def bitlen(x: int) -> int:
    return int(x).bit_length()

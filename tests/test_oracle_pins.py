"""The CPU oracle against its pins (no GPU), and the pages' co-rank search
(host model) against the printed trace, termination and the step bound."""
import numpy as np
import pytest

import oracle
import oracle_pins as P
from corank_model import bitlen, co_rank_search

pytestmark = pytest.mark.filterwarnings("error")


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_exhaustive_wider(orc):
    """m, n <= 6 over a 4-letter alphabet (44,100 pairs)."""
    P.pin_exhaustive_tiny(orc, max_len=6, alphabet=4)


def test_empty_sides(orc):
    A = np.array([-5, 0, 0, 7], dtype=np.int32)
    E = np.zeros(0, dtype=np.int32)
    assert np.array_equal(orc.merge_i32(A, E), A)
    assert np.array_equal(orc.merge_i32(E, A), A)
    assert orc.merge_i32(E, E).size == 0
    assert list(orc.co_rank_all(A, E)) == [0, 1, 2, 3, 4]
    assert list(orc.co_rank_all(E, A)) == [0, 0, 0, 0, 0]
    assert list(orc.co_rank_all(E, E)) == [0]


# ------------------------------------------------ host model of the search

def test_model_reproduces_printed_trace():
    g = P.load_golden("worked_example_corank.json")
    t = g["trace_co_rank_3"]
    r = co_rank_search(t["k"], g["A"], g["B"], record=True)
    assert r.i == t["returns_i"] and t["k"] - r.i == t["returns_j"]
    assert len(r.trace) == len(t["rows"])
    for got, want in zip(r.trace, t["rows"]):
        for key in ("iter", "i_low", "i", "j", "j_low", "verdict", "delta"):
            assert got[key] == want[key], (key, got, want)
    for k, i in zip(g["boundary_k"], g["boundary_i"]):
        assert co_rank_search(k, g["A"], g["B"]).i == i


def test_model_matches_oracle(orc):
    """The pages' search returns the oracle's co-rank for every k."""
    g = np.random.Generator(np.random.PCG64(23))
    for c in range(150):
        m, n = (int(x) for x in g.integers(0, 40, size=2))
        span = int(g.choice([2, 4, 1000]))
        A = np.sort(g.integers(0, span, size=m)).astype(np.int32)
        B = np.sort(g.integers(0, span, size=n)).astype(np.int32)
        I = orc.co_rank_all(A, B)
        Al, Bl = A.tolist(), B.tolist()
        for k in range(m + n + 1):
            assert co_rank_search(k, Al, Bl).i == I[k]


def test_floor_half_step_never_terminates():
    """With A=[1], B=[0], k=1 the answer is i=0.  Rounding the half-step down
    gives a zero step and the loop spins; rounding up returns at once."""
    assert co_rank_search(1, [1], [0]).i == 0
    r = co_rank_search(1, [1], [0], round_up=False, max_steps=1000)
    assert not r.finished


def test_step_bound():
    """At most bitlen(min(m, n)) adjustments before acceptance (merge_path.cu
    bounds the loop by the shorter input; its main() prints 22 for 2^21)."""
    g = np.random.Generator(np.random.PCG64(29))
    worst = 0
    for c in range(400):
        m, n = (int(x) for x in g.integers(0, 200, size=2))
        span = int(g.choice([2, 10, 1 << 20]))
        A = np.sort(g.integers(0, span, size=m)).tolist()
        B = np.sort(g.integers(0, span, size=n)).tolist()
        for k in range(0, m + n + 1, max(1, (m + n) // 17)):
            r = co_rank_search(k, A, B)
            assert r.steps <= bitlen(min(m, n)), (k, m, n, r.steps)
            worst = max(worst, r.steps - bitlen(min(m, n)))
    assert bitlen((1 << 21)) == 22


def test_unsorted_input_terminates():
    """Sortedness is a precondition; the search must still stop in range."""
    g = np.random.Generator(np.random.PCG64(31))
    for c in range(2000):
        m, n = (int(x) for x in g.integers(0, 30, size=2))
        A = g.integers(0, 8, size=m).tolist()
        B = g.integers(0, 8, size=n).tolist()
        k = int(g.integers(0, m + n + 1))
        r = co_rank_search(k, A, B, max_steps=4 * (bitlen(min(m, n)) + 2))
        assert r.finished
        assert max(0, k - n) <= r.i <= min(k, m)

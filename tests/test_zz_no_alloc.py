"""merge_i32_no_alloc, the entry point that allocates no device memory,
against merge_i32 (and the oracle) on two calls in a row, the second with a
smaller input: the static scratch keeps the first call's partition, and the
second call must not read any of it.  Merges that fit the device in one wave
of workgroups (up to about 8 million outputs) take the one-launch path and
use no scratch at all; the first pair keeps both calls above that, on the
scratch."""
import numpy as np
import pytest
import torch

import oracle
import ordered_merge_sorted_amd as om
from ordered_merge_sorted_amd.workloads import random_case

pytestmark = pytest.mark.gpu


def _dev(x):
    return torch.from_numpy(x).to("cuda:0")


@pytest.mark.parametrize("first,second", [
    # 16.8M outputs (4,097 co-ranks in the scratch), then 9M (2,199): both
    # through the partition array
    ((16, (1 << 23) + 5, (1 << 23) - 3, -(1 << 31), (1 << 31) - 1), (17, 5000011, 4000037, -100, 100)),
    # 16.8M outputs: full 4,096-output segments (4,097 co-ranks); then 120k
    ((11, (1 << 23) + 123, (1 << 23) - 77, -(1 << 31), (1 << 31) - 1), (12, 70001, 50003, -40, 40)),
    # many ties, then a tiny ragged case with one empty side
    ((13, 3000017, 2999999, -1000, 1000), (14, 4099, 0, -5, 5)),
])
def test_no_alloc_matches_merge_i32_on_two_calls(first, second):
    torch.cuda.set_device(0)
    for seed, m, n, lo, hi in (first, second):
        A, B = random_case(seed, m, n, lo=lo, hi=hi)
        a, b = _dev(A), _dev(B)
        ref = om.merge_i32(a, b)
        got = torch.full((m + n,), -7, dtype=torch.int32, device="cuda:0")
        om.merge_i32_no_alloc(a, b, out=got)
        torch.cuda.synchronize()
        print("no-alloc merge seed=%d m=%d n=%d" % (seed, m, n), flush=True)
        assert torch.equal(got, ref), (seed, m, n)
        assert np.array_equal(got.cpu().numpy(), oracle.merge_i32(A, B)), (seed, m, n)


def test_no_alloc_on_a_side_stream():
    torch.cuda.set_device(0)
    A, B = random_case(15, 200003, 100001, lo=-300, hi=300)
    a, b = _dev(A), _dev(B)
    s = torch.cuda.Stream()
    got = torch.empty(A.size + B.size, dtype=torch.int32, device="cuda:0")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        om.merge_i32_no_alloc(a, b, out=got, stream=s)
    s.synchronize()
    assert np.array_equal(got.cpu().numpy(), oracle.merge_i32(A, B))

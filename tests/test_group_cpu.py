"""Group semantics that need no GPU: the aggregation rule as a pure function
(sorting, buckets, the 4x run rule, isolation) against a brute-force
restatement, and the group depth / error bookkeeping of arGroupStart /
arGroupEnd."""
import random

import pytest


@pytest.fixture(scope="module")
def B():
    import os
    from ring_allreduce_reduction_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from ring_allreduce_reduction_amd.build import build
        build()
    binding.lib()
    return binding


def _expected(keys, nbytes, isolate):
    """The rule spelled out: largest first (stable), buckets by key ascending,
    runs that start at a task and take followers while 4*bytes > the start's."""
    idx = sorted(range(len(keys)), key=lambda i: -nbytes[i])      # sorted() is stable
    launches = []
    for key in sorted(set(keys)):
        lst = [i for i in idx if keys[i] == key]
        i = 0
        while i < len(lst):
            run = [lst[i]]
            j = i + 1
            if not isolate[lst[i]]:
                while j < len(lst) and not isolate[lst[j]] and 4 * nbytes[lst[j]] > nbytes[lst[i]]:
                    run.append(lst[j])
                    j += 1
            launches.append(run)
            i = j
    return launches


def _launches(order, launch_of):
    out = []
    for t in order:
        if not out or launch_of[t] != launch_of[out[-1][0]]:
            out.append([])
        out[-1].append(t)
    return out


def test_within_4x_and_sorting(B):
    # sizes 100, 30, 26, 25, 7 in one bucket: 100 takes 30 and 26 (4*25 = 100
    # is not more); 25 then starts a run that takes 7 (4*7 = 28 > 25)
    order, launch_of, n = B.arGroupAggregate([0] * 5, [25, 100, 7, 26, 30])
    assert n == 2
    assert _launches(order, launch_of) == [[1, 4, 3], [0, 2]]
    assert _launches(order, launch_of) == _expected([0] * 5, [25, 100, 7, 26, 30], [0] * 5)


def test_buckets_and_isolation(B):
    keys = [3, 1, 3, 1, 2]
    nbytes = [64, 64, 64, 64, 64]
    order, launch_of, n = B.arGroupAggregate(keys, nbytes)
    assert _launches(order, launch_of) == [[1, 3], [4], [0, 2]]        # buckets ascending, call order kept
    order, launch_of, n = B.arGroupAggregate(keys, nbytes, isolate=[0, 1, 0, 0, 0])
    assert _launches(order, launch_of) == [[1], [3], [4], [0, 2]]


@pytest.mark.parametrize("seed", range(40))
def test_random_against_brute_force(B, seed):
    rng = random.Random(seed)
    n = rng.randint(1, 40)
    keys = [rng.randint(0, 4) for _ in range(n)]
    nbytes = [rng.choice([1, 2, 3, 4, 5, 16, 17, 64, 65, 255, 256, 1000, 4096]) for _ in range(n)]
    isolate = [int(rng.random() < 0.2) for _ in range(n)]
    order, launch_of, nl = B.arGroupAggregate(keys, nbytes, isolate)
    want = _expected(keys, nbytes, isolate)
    assert _launches(order, launch_of) == want and nl == len(want)
    assert sorted(order) == list(range(n))


def test_empty_and_errors(B):
    assert B.arGroupAggregate([], []) == ([], [], 0)
    import ctypes
    assert B.lib().arGroupAggregate(-1, None, None, None, None, None, ctypes.byref(ctypes.c_int())) \
        == B.arInvalidArgument


def test_group_depth_bookkeeping(B):
    L = B.lib()
    assert L.arGroupEnd() == B.arInvalidUsage            # not in a group
    assert L.arGroupStart() == B.arSuccess
    assert L.arGroupStart() == B.arSuccess               # nested
    assert L.arGroupEnd() == B.arSuccess                 # inner end launches nothing
    assert L.arGroupEnd() == B.arSuccess                 # outer end: no comm joined
    assert L.arGroupEnd() == B.arInvalidUsage


def test_group_error_reported_at_end(B):
    import ctypes
    L = B.lib()
    ptrs = (ctypes.c_void_p * 1)(0)
    assert L.arGroupStart() == B.arSuccess
    assert L.arAllReduce(None, ptrs, ptrs, 4, B.arFloat32, B.arSum, None) == B.arInvalidArgument
    assert L.arGroupEnd() == B.arInvalidArgument         # the group's first error
    assert L.arGroupStart() == B.arSuccess               # and the next group starts clean
    assert L.arGroupEnd() == B.arSuccess

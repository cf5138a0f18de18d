"""Rings and trees cut into workgroups at any group size (arDebugGroupSize):
every edge between two groups is a device-coherent hop, every other one a
handoff inside a workgroup, and the result must not depend on which is
which.  The pages' definition of the result, every rank holding the same
full reduction ["NCCL 原始碼解讀：一個 AllReduce 的 GPU 旅程", ch.1 §1.3],
is checked bit for bit against the oracle run on the plan that ran, at
group sizes that leave a ragged last group, one member per workgroup
(every edge between workgroups), and on rings short enough to fit one
workgroup otherwise."""
import pytest
import torch

pytestmark = pytest.mark.gpu

CASES = [
    # n, members per workgroup at most, count (fp32), channels
    (8, 3, 300007, 4),        # groups 3, 3, 2
    (8, 1, 70001, 2),         # every edge between workgroups
    (16, 5, 1 << 20, 16),     # groups 4 x 4 (balanced from 5)
    (24, 7, 1 << 18, 8),      # groups 6 x 4
    (72, 12, 1 << 20, 64),    # the 72-rank x 4 MiB workload, 6 groups
    (72, 1, 1 << 18, 8),      # 72 workgroups per lane
]


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ring_allreduce_reduction_amd import binding
    binding.lib()
    return binding


@pytest.fixture(scope="module")
def gu():
    import gpu_util
    return gpu_util


@pytest.mark.parametrize("proto", ["simple", "ll", "ll128"])
@pytest.mark.parametrize("algo", ["ring", "tree"])
@pytest.mark.parametrize("case", CASES, ids=["n%d-gs%d" % (c[0], c[1]) for c in CASES])
def test_group_size_parity(B, gu, case, proto, algo):
    n, gs, count, nch = case
    with B.Comm(n, nch, proto, algo) as comm:
        B.arSetDebug(comm.handle, B.arDebugGroupSize, gs)
        plan = comm.plan(count, "float32")
        assert plan["ranksPerGroup"] <= gs
        assert -(-n // plan["ranksPerGroup"]) > 1
        gu.parity_case(n, count, "float32", "sum", proto, nch, seed=gs * 100 + n, comm=comm)
        # back to whole workgroups where the ring fits one: the counters that
        # crossed workgroups carry over into LDS handoffs
        B.arSetDebug(comm.handle, B.arDebugGroupSize, 0)
        gu.parity_case(n, count, "float32", "sum", proto, nch, seed=gs * 100 + n + 1, comm=comm)
        if algo == "ring":
            gu.parity_case(n, 4099, "bfloat16", "max", proto, nch, seed=7, comm=comm)


def test_group_size_knob_range(B):
    """Values outside 0..16 are refused (host only, nothing launched)."""
    with B.Comm(4, 1, "simple") as comm:
        for bad in (-1, 17):
            with pytest.raises(B.ArError):
                B.arSetDebug(comm.handle, B.arDebugGroupSize, bad)

"""The Simple ring with its FIFO slots in LDS (the kernels for rings inside
one workgroup, and the edges inside each group of a longer ring).  The slot
location never changes a result, so every case checks the pages' definition
of the result ["NCCL 原始碼解讀：一個 AllReduce 的 GPU 旅程", ch.1 §1.3: every
rank holds the same full reduction] bit for bit against the oracle run on the
plan that ran, and that the plan put the slots where it says.  Calls with LDS
and device FIFOs alternate on one comm: the LDS calls start every edge at
step 0 and leave the comm's device counters as they found them, so the
device-FIFO calls around them must still meet at tail == head."""
import pytest
import torch

pytestmark = pytest.mark.gpu


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


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.lib()
    return oracle


@pytest.mark.parametrize("n,count,nch", [(2, 1000003, 8), (5, 777777, 16), (8, 300007, 4), (16, 262147, 64),
                                         (8, 1 << 22, 64), (3, 5, 1)])
def test_plan_reports_lds_and_parity_both_ways(B, gu, n, count, nch):
    with B.Comm(n, nch, "simple") as comm:
        plan = comm.plan(count, "float32")
        assert plan["ldsFifoBytes"] == n * plan["nSlots"] * plan["stepBytes"] > 0
        assert plan["deviceBytes"] == pytest.approx(2.0 * n * count * 4)
        gu.parity_case(n, count, "float32", "sum", "simple", nch, seed=n, comm=comm)
        B.arSetDebug(comm.handle, B.arDebugLdsFifo, 0)
        plan0 = comm.plan(count, "float32")
        assert plan0["ldsFifoBytes"] == 0 and plan0["deviceBytes"] == plan0["modelBytes"]
        gu.parity_case(n, count, "float32", "sum", "simple", nch, seed=n + 1, comm=comm)


def test_lds_and_device_fifo_calls_alternate_on_one_comm(B, gu):
    """Device-FIFO calls carry their counters across calls; LDS calls in
    between must not disturb them (and an LL call reuses the same edges)."""
    n, nch = 8, 16
    with B.Comm(n, nch, "simple") as comm:
        for i, (lds, proto, count) in enumerate([(1, "simple", 1 << 20), (0, "simple", 300007), (1, "simple", 4099),
                                                 (0, "simple", 1 << 20), (1, "ll", 200003), (1, "simple", 777),
                                                 (0, "simple", 65541), (1, "simple", 1 << 21)]):
            B.arSetDebug(comm.handle, B.arDebugLdsFifo, lds)
            plan = gu.parity_case(n, count, "float32", "sum", proto, nch, seed=100 + i, comm=comm)[0]
            assert (plan["ldsFifoBytes"] > 0) == (lds == 1 and proto == "simple")


@pytest.mark.parametrize("depth", [2, 3, 4, 8])
@pytest.mark.parametrize("n", [4, 16])
def test_lds_fifo_depths(B, gu, n, depth):
    """arDebugSlots sets the LDS depth too; the slot shrinks until N x depth
    slots fit a workgroup's LDS."""
    count = 1 << 21
    with B.Comm(n, 32, "simple") as comm:
        B.arSetDebug(comm.handle, B.arDebugSlots, depth)
        plan = comm.plan(count, "float32")
        assert plan["nSlots"] == depth and plan["ldsFifoBytes"] == n * depth * plan["stepBytes"]
        assert plan["ldsFifoBytes"] <= 160 * 1024
        gu.parity_case(n, count, "float32", "sum", "simple", 32, seed=depth, comm=comm)
        gu.parity_case(n, 123457, "bfloat16", "sum", "simple", 32, seed=depth + 1, comm=comm)


@pytest.mark.parametrize("slot_kib", [1, 2, 4])
def test_lds_fifo_slot_sizes_and_lane_sets(B, gu, slot_kib):
    n, nch, count = 8, 8, 3000017
    with B.Comm(n, nch, "simple") as comm:
        B.arSetDebug(comm.handle, B.arDebugSimpleSlotKiB, slot_kib)
        for sets in (0, 5):   # 5 persistent workgroups run every (channel, lane) pair in turn
            B.arSetDebug(comm.handle, B.arDebugLaneSets, sets)
            plan = gu.parity_case(n, count, "float32", "sum", "simple", nch, seed=slot_kib + sets, comm=comm)[0]
            assert plan["ldsFifoBytes"] > 0 and plan["stepBytes"] <= slot_kib * 1024


@pytest.mark.parametrize("inplace,offset", [(True, 0), (False, 1), (True, 1)])
@pytest.mark.parametrize("dtype,op", [("float32", "sum"), ("float16", "min"), ("int32", "max"), ("uint64", "probe")])
def test_lds_fifo_inplace_unaligned_types(B, gu, inplace, offset, dtype, op):
    gu.parity_case(8, 262151, dtype, op, "simple", 16, seed=7, inplace=inplace, offset=offset)


def test_lds_fifo_halves(B, gu, orc):
    from test_gpu_rs_ag import ag_case, rs_case
    for n, count in [(8, 65541), (16, 4099), (3, 1 << 18)]:
        with B.Comm(n, 16, "simple") as comm:
            rs_case(B, gu, orc, n, count, "float32", "sum", "simple", 16, seed=n, comm=comm)
            ag_case(B, gu, orc, n, count, "bfloat16", "simple", 16, seed=n, comm=comm)


def test_lds_fifo_grouped_launch(B, gu):
    from test_gpu_group import run_group
    with B.Comm(8, 16, "simple", "ring") as comm:
        plans = run_group(B, gu, comm, [(c, "float32", "sum", False, i)
                                        for i, c in enumerate([4096, 4100, 5000, 65537, 70000, 1 << 20])], "lds")
        assert max(p["tasksInLaunch"] for p in plans) >= 2
        assert all(p["ldsFifoBytes"] > 0 for p in plans)


@pytest.mark.parametrize("n,count,nch,dtype", [(17, 4096, 64, "float32"), (32, 1027, 64, "float32"),
                                               (72, 1024, 64, "float32"), (40, 2048, 64, "bfloat16"),
                                               (128, 1024, 64, "int32"), (64, 16384, 64, "float32"),
                                               (24, 32771, 64, "float16")])
def test_tree_cut_into_workgroups_keeps_inside_edges_in_lds(B, gu, n, count, nch, dtype):
    """A Simple tree past 16 ranks: the edges inside each workgroup in LDS,
    the edges between workgroups in device memory with carried counters.  The
    plan says so, the result is the oracle's either way, and calls with and
    without the LDS FIFOs alternate on one comm (the device edges' counters
    must still meet at tail == head)."""
    from ring_allreduce_reduction_amd import binding
    with B.Comm(n, nch, "simple", "tree") as comm:
        plan = comm.plan(count, dtype)
        gs = plan["ranksPerGroup"]
        assert plan["algo"] == binding.arAlgoTree and gs < n, plan
        assert plan["ldsFifoBytes"] == 2 * gs * plan["nSlots"] * plan["stepBytes"] > 0, plan
        esz = 2 if dtype in ("bfloat16", "float16") else 4
        assert plan["deviceBytes"] > 2.0 * n * count * esz   # edges between workgroups move bytes too
        for i, lds in enumerate([1, 0, 1, 1, 0]):
            B.arSetDebug(comm.handle, B.arDebugLdsFifo, lds)
            p = comm.plan(count, dtype)
            assert (p["ldsFifoBytes"] > 0) == bool(lds), p
            gu.parity_case(n, count, dtype, "sum", "simple", nch, seed=n + i, comm=comm)
        gu.parity_case(n, count, "uint64", "probe", "simple", nch, comm=comm)

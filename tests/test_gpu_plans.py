"""GPU parity on the plans three planner rules produce, with the rule itself
checked on the plan: rings of fewer than 8 ranks spread a short chunk over
up to 8 wavefronts per CU, a tree whose lanes the FIFOs cap keeps its
largest slot, and a ring cut into workgroups keeps at most 24 of its
wavefronts on a CU (a tree too), its inside FIFOs in LDS and a slot that
fits its chunk.
Bit for bit against the oracle on every rank."""
import pytest
import torch

pytestmark = pytest.mark.gpu

MiB = 1 << 20


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
def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("n,nbytes", [(2, 2 * MiB), (2, 4 * MiB), (2, 8 * MiB), (3, 4 * MiB), (4, 8 * MiB)])
def test_small_ring_spreads_short_chunks(B, gu, cus, n, nbytes):
    count = nbytes // 4
    plan, _, _ = gu.parity_case(n, count, "float32", "sum", "simple", 64, seed=n)
    lanes, slot, nch = plan["lanesPerChannel"], plan["stepBytes"], plan["nChannels"]
    assert slot < 8192, plan                                  # a halved slot ...
    assert nch * lanes > cus, plan                            # ... past one workgroup per CU
    assert nch * lanes <= cus * (8 // n), plan                # ... within 8 wavefronts per CU
    chunk = nbytes // nch // n                                # one loop: the chunk is a rank's share
    assert lanes * slot >= chunk // 2, plan                   # a lane's share is about one slot


@pytest.mark.parametrize("n,nbytes", [(8, 8 * MiB), (16, 4 * MiB), (3, 16 * MiB), (4, 16 * MiB)])
def test_fifo_capped_tree_keeps_its_slot(B, gu, n, nbytes):
    count = nbytes // 4
    plan, _, _ = gu.parity_case(n, count, "float32", "sum", "simple", 64, algo="tree", seed=n + 1)
    lanes, slot, nch = plan["lanesPerChannel"], plan["stepBytes"], plan["nChannels"]
    want = 4096                                               # the tree's largest Simple slot,
    if plan["ldsFifoBytes"]:                                  # or the largest whose 2N FIFOs fit LDS
        while 2 * n * plan["nSlots"] * want + 512 > 160 * 1024:
            want //= 2
        assert plan["ldsFifoBytes"] == 2 * n * plan["nSlots"] * slot
    assert slot == want, plan
    assert lanes * slot < nbytes // nch, plan                 # shares span several slots


@pytest.mark.parametrize("n,nbytes", [(76, 8 * MiB), (72, 8 * MiB), (52, 8 * MiB), (100, 2 * MiB)])
def test_ring_cut_into_workgroups_plan(B, gu, cus, n, nbytes):
    # sizes whose earlier plans fell into one-member groups (76 ranks), 4 KiB
    # slots for 1.8 KiB chunks (72), or two 13-member workgroups per CU (52,
    # 100): each took 1.4-3.8x the time of the plan checked here
    count = nbytes // 4
    plan, _, _ = gu.parity_case(n, count, "float32", "sum", "simple", 64, seed=n + 2)
    gs, wg, slot = plan["ranksPerGroup"], plan["workgroups"], plan["stepBytes"]
    assert 1 < gs <= 16 and plan["ldsFifoBytes"] > 0, plan
    assert -(-wg // cus) * gs <= 24, plan                     # ring wavefronts per CU
    chunk = nbytes // plan["nChannels"] // n                  # one loop: a rank's share of a channel
    assert chunk <= slot and (slot == 1024 or slot // 2 < chunk), plan


@pytest.mark.parametrize("n,nbytes,nch", [(40, 128 << 10, 4), (52, 128 << 10, 4), (72, 4 * MiB, 16)])
def test_tree_cut_into_workgroups_waves_per_cu(B, gu, cus, n, nbytes, nch):
    # 40 and 52 ranks once ran two 13-14-member workgroups on a CU (1.5x the
    # time of the plan checked here)
    plan, _, _ = gu.parity_case(n, nbytes // 4, "float32", "sum", "simple", nch, algo="tree", seed=n + 3)
    gs, wg = plan["ranksPerGroup"], plan["workgroups"]
    assert 1 < gs <= 16, plan
    assert -(-wg // cus) * gs <= 24, plan
    if plan["ldsFifoBytes"] == 0:                               # device FIFOs: taken at depth 4
        assert plan["nSlots"] == 4, plan
    else:                                                       # LDS FIFOs: as deep as still fits
        assert plan["ldsFifoBytes"] == 2 * gs * plan["nSlots"] * plan["stepBytes"] <= 160 * 1024, plan


def test_deeper_fifos_provisioned_on_first_call_of_a_nonblocking_stream(B, gu):
    # A ring cut into workgroups takes depth-4 FIFOs where they fit LDS; its
    # first call provisions the device FIFOs of its edges between workgroups
    # at that depth.  The clear of the new FIFOs must be complete before the
    # kernel runs on a stream that does not wait for the null stream (a run
    # that raced it once ran a later call into the wait bound).
    from ring_allreduce_reduction_amd import inputs as gen
    n, count = 72, 1 << 18
    xs = gen.make_inputs(n, count, "float32", seed=5)
    sends = [gu.to_device(x, "float32") for x in xs]
    recvs = [torch.empty_like(t) for t in sends]
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with B.Comm(n, 64, "simple", "ring") as comm:
        plan = comm.plan(count, "float32")
        assert plan["nSlots"] == 4 and plan["ldsFifoBytes"] == plan["ranksPerGroup"] * 4 * plan["stepBytes"], plan
        for _ in range(64):
            B.arAllReduce(comm.handle, sends, recvs, stream=s)
        torch.cuda.synchronize()
        assert comm.async_error() == B.arSuccess
        want = gu.expected(xs, "float32", "sum", plan)
        for r in range(n):
            gu.assert_bits_equal(gu.to_host_raw(recvs[r], "float32"), want, "float32", "rank %d" % r)


def test_small_ring_ragged_and_16bit(B, gu):
    # the spread plan on a count no slot divides, and on both 16-bit types
    gu.parity_case(2, (4 * MiB) // 4 + 12345, "float32", "sum", "simple", 64, seed=5)
    gu.parity_case(3, (4 * MiB) // 2 + 777, "bfloat16", "sum", "simple", 64, seed=6)
    gu.parity_case(4, (8 * MiB) // 2 + 1, "float16", "sum", "simple", 64, seed=7)


@pytest.mark.parametrize("n,proto,algo", [(24, "simple", "ring"), (24, "ll128", "ring"), (40, "ll", "tree"),
                                          (72, "simple", "tree")])
def test_cooperative_and_plain_launches_agree(B, gu, orc, n, proto, algo):
    """Rings and trees cut into workgroups run plainly launched by default;
    the cooperative launch (arDebugCooperative = 1) runs the same grid and
    gives the same bits, both equal to the oracle on the plan."""
    with B.Comm(n, 16, proto, algo) as comm:
        for coop in (1, 0):
            B.arSetDebug(comm.handle, B.arDebugCooperative, coop)
            plan, _, _ = gu.parity_case(n, 70001, "float32", "sum", proto, 16, seed=n + coop, comm=comm)
            assert plan["ranksPerGroup"] < n


def test_fifo_footprint_follows_the_protocols(B, gu, orc):
    """A comm provisions the FIFOs of the protocols it may run, each at the
    depth it runs with: N x lanesMax workers x depth x the largest slot (8 KiB
    Simple, 2 KiB LL, 4 KiB LL128) plus 256 bytes of counters each."""
    n = 8
    workers = n * (32768 // n)
    simple = workers * (2 * 8192 + 256)
    ll = workers * (8 * 2048 + 256)
    ll128 = workers * (8 * 4096 + 256)
    with B.Comm(n, 16, "simple") as comm:
        assert comm.footprint() == 256 + simple
        gu.parity_case(n, 300007, "float32", "sum", "simple", 16, seed=1, comm=comm)
        comm.set_config("ll", 16)                         # a protocol switched to is provisioned then
        assert comm.footprint() == 256 + simple + ll
        gu.parity_case(n, 300007, "float32", "sum", "ll", 16, seed=2, comm=comm)
        B.arSetDebug(comm.handle, B.arDebugSlots, 4)      # Simple deeper (2 -> 4): re-provisioned from zero;
        assert comm.footprint() == 256 + workers * (4 * 8192 + 256) + ll   # LL shallower (8 -> 4): kept
        gu.parity_case(n, 300007, "float32", "sum", "ll", 16, seed=3, comm=comm)
        gu.parity_case(n, 300007, "float32", "sum", "simple", 16, seed=4, comm=comm)
    with B.Comm(n, 64, "auto", "auto") as comm:
        assert comm.footprint() == 256 + simple + ll + ll128
        assert comm.footprint() < (5 << 29)                # 2.5 GiB, every protocol

"""GPU parity: the HIP ring AllReduce, called through the C ABI, against the
CPU oracle on the same seeded inputs, bit for bit on every rank.  Sizes span
several FIFO slots, several lanes and ragged tails; the edge cases are the
empty call, one rank, two ranks, in place, unaligned buffers, repeated calls
on one comm across protocols, and rings cut over several workgroups."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

PROTOS = ["simple", "ll", "ll128"]


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


# ---------------------------------------------------------------- pages' values

@pytest.mark.parametrize("proto", PROTOS)
def test_worked_example(B, gu, proto):
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")))
    xs = [np.array(v, dtype=np.float32) for v in g["inputs"]]
    gu.note("worked example proto=%s" % proto)
    with B.Comm(4, 1, proto) as comm:
        sends = [gu.to_device(x, "float32") for x in xs]
        recvs = [gu.empty_like_sentinel(2, "float32") for _ in range(4)]
        gu.run_ring(comm, sends, recvs, "float32", "sum")
        for r in range(4):
            assert recvs[r].cpu().tolist() == g["expected_every_rank"]


@pytest.mark.parametrize("n", [2, 8, 16])
def test_rank_marker(B, gu, n):
    from ring_allreduce_reduction_amd import inputs as gen
    count = (1 << 20) + 3
    xs = gen.rank_marker_inputs(n, count)
    gu.note("rank marker n=%d" % n)
    with B.Comm(n, 8, "simple") as comm:
        sends = [gu.to_device(x, "float32") for x in xs]
        recvs = [gu.empty_like_sentinel(count, "float32") for _ in range(n)]
        gu.run_ring(comm, sends, recvs, "float32", "sum")
        for r in range(n):
            assert recvs[r][0].item() == n * (n - 1) // 2
            assert torch.count_nonzero(recvs[r][1:]).item() == 0


# ---------------------------------------------------------------- parity sweep

@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("n,count,nch", [
    (2, 1, 1), (2, 4099, 2), (3, 777, 1), (4, 2, 1), (4, 100003, 3),
    (8, 12345, 4), (8, 262147, 16), (5, 1 << 18, 7), (16, 70001, 5)])
def test_fp32_sum_parity(B, gu, proto, n, count, nch):
    gu.parity_case(n, count, "float32", "sum", proto, nch, seed=n + count)


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("dtype", ["int32", "float32", "float16", "bfloat16"])
@pytest.mark.parametrize("op", ["sum", "max", "min"])
def test_dtype_op_parity(B, gu, proto, dtype, op):
    gu.parity_case(6, 50021, dtype, op, proto, 4, seed=17)


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("n", [2, 3, 8, 15])
def test_order_probe_on_device(B, gu, proto, n):
    # uint64 acc*16 + x: the oracle's probe digits are pinned by hand-derived
    # chunk indices; bit equality here means the device visits ranks in the
    # same order for every element.
    gu.parity_case(n, 3001, "uint64", "probe", proto, 3)


@pytest.mark.parametrize("proto", PROTOS)
def test_in_place(B, gu, proto):
    gu.parity_case(8, 100001, "float32", "sum", proto, 4, seed=3, inplace=True)
    gu.parity_case(8, 100001, "bfloat16", "sum", proto, 4, seed=3, inplace=True)


@pytest.mark.parametrize("proto", ["simple", "ll"])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
def test_unaligned_buffers(B, gu, proto, dtype):
    gu.parity_case(4, 30011, dtype, "sum", proto, 3, seed=5, offset=1)


@pytest.mark.parametrize("slot_kib", [1, 2, 4])
@pytest.mark.parametrize("direct", [0, 1])
def test_simple_slot_and_direct_variants(B, gu, slot_kib, direct):
    with B.Comm(8, 16, "simple") as comm:
        B.arSetDebug(comm.handle, B.arDebugSimpleSlotKiB, slot_kib)
        B.arSetDebug(comm.handle, B.arDebugDirect, direct)
        for count, nch, lanes in [(300007, 5, 0), (1 << 20, 16, 3), (4099, 2, 0)]:
            B.arSetDebug(comm.handle, B.arDebugLanes, lanes)
            gu.parity_case(8, count, "float32", "sum", "simple", nch, seed=count, comm=comm)
        B.arSetDebug(comm.handle, B.arDebugLanes, 0)
        gu.parity_case(8, 100003, "bfloat16", "sum", "simple", 4, seed=1, comm=comm, inplace=True)
        gu.parity_case(5, 77777, "int32", "max", "simple", 3, seed=2, comm=None)


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("sets", [1, 3, 7])
def test_workgroups_running_several_lanes(B, gu, proto, sets):
    # fewer workgroups than (channel, lane) pairs: workgroup L runs pairs
    # L, L + sets, ... on one FIFO set, its steps continuing across pairs
    with B.Comm(8, 16, proto) as comm:
        B.arSetDebug(comm.handle, B.arDebugLaneSets, sets)
        for count, nch in [(300007, 5), (1 << 20, 16), (4099, 2)]:
            plan, _, _ = gu.parity_case(8, count, "float32", "sum", proto, nch, seed=count + sets, comm=comm)
            assert plan["workgroups"] <= sets
        gu.parity_case(8, 100003, "bfloat16", "sum", proto, 4, seed=sets, comm=comm, inplace=True)
        gu.parity_case(8, 3001, "uint64", "probe", proto, 3, comm=comm)
        B.arSetDebug(comm.handle, B.arDebugLaneSets, 0)
        gu.parity_case(8, 300007, "float32", "sum", proto, 5, seed=9, comm=comm)


@pytest.mark.parametrize("slot_kib", [2, 4])
def test_ll128_slot_variants(B, gu, slot_kib):
    # LL128 slots of 2 or 4 KiB of wire (16 or 32 lines of 120 payload bytes)
    with B.Comm(8, 16, "ll128") as comm:
        B.arSetDebug(comm.handle, B.arDebugLL128SlotKiB, slot_kib)
        for count, nch in [(300007, 5), (1 << 20, 16), (4099, 2), (777, 1)]:
            plan, _, _ = gu.parity_case(8, count, "float32", "sum", "ll128", nch, seed=count, comm=comm)
            assert plan["stepBytes"] == slot_kib * 1024
        gu.parity_case(8, 100003, "bfloat16", "sum", "ll128", 4, seed=1, comm=comm, inplace=True)
        gu.parity_case(8, 3001, "uint64", "probe", "ll128", 3, comm=comm)
        gu.parity_case(8, 50021, "int32", "min", "ll128", 3, seed=2, comm=comm)
    with B.Comm(24, 4, "ll128") as comm:   # a ring of two workgroups
        B.arSetDebug(comm.handle, B.arDebugLL128SlotKiB, slot_kib)
        gu.parity_case(24, 40009, "float32", "sum", "ll128", 4, seed=24, comm=comm)


def test_ll128_needs_128_byte_alignment(B, gu):
    from ring_allreduce_reduction_amd import inputs as gen
    xs = gen.make_inputs(4, 1000, "float32")
    with B.Comm(4, 2, "ll128") as comm:
        sends = [gu.to_device(x, "float32", offset_elems=1) for x in xs]
        recvs = [gu.empty_like_sentinel(1000, "float32", offset_elems=1) for _ in range(4)]
        with pytest.raises(B.ArError) as e:
            B.arAllReduce(comm.handle, sends, recvs, op=B.arSum)
        assert e.value.code == B.arInvalidUsage
    # auto never picks LL128 for such buffers and still gets the right answer
    with B.Comm(4, 2, "auto") as comm:
        plan = comm.plan(1000, "float32", aligned128=False)
        assert plan["proto"] != B.arProtoLL128


def test_repeated_calls_across_protocols(B, gu):
    # one comm, protocols and sizes interleaved: the monotonic FIFO counters
    # and per-protocol flags must carry over correctly from call to call
    with B.Comm(8, 16, "simple") as comm:
        for i, (proto, count, nch) in enumerate([("simple", 70000, 16), ("ll", 5000, 2), ("ll128", 90001, 8),
                                                 ("simple", 1, 1), ("ll", 120000, 16), ("ll128", 7, 3),
                                                 ("simple", 300001, 5), ("ll", 5000, 2), ("ll128", 90001, 8)]):
            gu.parity_case(8, count, "float32", "sum", proto, nch, seed=100 + i, comm=comm)


def test_empty_and_single_rank(B, gu):
    from ring_allreduce_reduction_amd import inputs as gen
    with B.Comm(4, 2, "simple") as comm:
        t = [torch.zeros(0, device="cuda") for _ in range(4)]
        B.arAllReduce(comm.handle, t, t, count=0, dtype=B.arFloat32)
    gu.parity_case(1, 12345, "float32", "sum", "simple", 1)
    x = gen.make_inputs(1, 1000, "bfloat16")
    gu.parity_case(1, 1000, "bfloat16", "max", "ll", 1, inputs=x, inplace=True)


@pytest.mark.parametrize("proto", ["simple", "ll128", "ll"])
@pytest.mark.parametrize("n", [17, 24, 40])
def test_rings_across_workgroups(B, gu, proto, n):
    gu.parity_case(n, 40009, "float32", "sum", proto, 4, seed=n)


@pytest.mark.parametrize("algo", ["ring", "tree"])
@pytest.mark.parametrize("proto", ["simple", "ll128", "ll"])
def test_grid_too_large_for_co_residency_halves_channels(B, gu, algo, proto):
    # 72 ranks on 64 channels: the LL kernels (and the tree's LL128) cannot
    # keep one lane per channel resident; the call runs on fewer channels and
    # reports them, and matches the oracle for that count
    with B.Comm(72, 64, proto, algo) as comm:
        plan, _, _ = gu.parity_case(72, 1 << 16, "float32", "sum", proto, 64, seed=72, comm=comm)
        assert 1 <= plan["nChannels"] <= 64 and plan["ranksPerGroup"] <= 16


@pytest.mark.parametrize("proto", ["simple", "ll128", "ll"])
@pytest.mark.parametrize("n", [24, 72])
def test_rings_across_xcds(B, gu, proto, n):
    # the workgroups of one (channel, lane) on consecutive ids, i.e. on
    # different XCDs (different L2s): the edges between them must be
    # device-coherent, not merely coherent within one L2
    with B.Comm(n, 16, proto) as comm:
        B.arSetDebug(comm.handle, B.arDebugGroupSpread, 1)
        for count, nch, dtype, op in [(40009, 4, "float32", "sum"), (300007, 16, "bfloat16", "sum"),
                                      (7001, 2, "int32", "max")]:
            plan, _, _ = gu.parity_case(n, count, dtype, op, proto, nch, seed=count + n, comm=comm)
            assert plan["ranksPerGroup"] < n
        gu.parity_case(n, 3001, "uint64", "probe", proto, 3, comm=comm)
        for algo in ("tree", "ring"):
            comm.set_algo(algo)
            gu.parity_case(n, 100003, "float32", "sum", proto, 8, seed=7, comm=comm)


def test_invalid_arguments_enqueue_nothing(B, gu):
    from ring_allreduce_reduction_amd import inputs as gen
    xs = gen.make_inputs(4, 256, "float32")
    with B.Comm(4, 2, "simple") as comm:
        sends = [gu.to_device(x, "float32") for x in xs]
        recvs = [gu.empty_like_sentinel(256, "float32") for _ in range(4)]
        L = B.lib()
        import ctypes
        sp, rp = B._ptrs(sends), B._ptrs(recvs)
        assert L.arAllReduce(comm.handle, sp, rp, 256, 7, 0, None) == B.arInvalidArgument        # dtype
        assert L.arAllReduce(comm.handle, sp, rp, 256, 1, 9, None) == B.arInvalidArgument        # op
        assert L.arAllReduce(comm.handle, sp, rp, 256, 1, B.arProbe, None) == B.arInvalidArgument
        dup = B._ptrs([recvs[0], recvs[0], recvs[2], recvs[3]])
        assert L.arAllReduce(comm.handle, sp, dup, 256, 1, 0, None) == B.arInvalidArgument     # shared output
        cross = B._ptrs([sends[1], recvs[1], recvs[2], recvs[3]])
        assert L.arAllReduce(comm.handle, sp, cross, 256, 1, 0, None) == B.arInvalidArgument   # output on input
        nul = (ctypes.c_void_p * 4)(0, 0, 0, 0)
        assert L.arAllReduce(comm.handle, nul, rp, 256, 1, 0, None) == B.arInvalidArgument
        torch.cuda.synchronize()
        for r in recvs:   # nothing ran
            assert torch.all(r.view(torch.int32) == -1).item()

"""GPU parity on every branch of the loop / chunk walk, element by element.

The pages walk a channel's share in loops of nRanks chunks and shrink only
the last, partial loop ["NCCL 原始碼解讀：一個 AllReduce 的 GPU 旅程", ch.2
§2.3, getNextSendAddr: curLoop full loops of nRanks x chunk, then the chunk
recomputed from what remains].  Each case here gives every channel at least
two full loops plus a ragged shrunk last loop, for every protocol, in fp32,
bf16 and the uint64 order probe, and compares every rank's output with the
oracle run on the same plan.  ReduceScatter / AllGather blocks that span
several chunks cover the halves' chunk loop the same way."""
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


def loops_per_channel(orc, n, count, dtype, nch, chunk):
    """Index of the last loop of every channel (2 = two full loops and a
    third, shrunk one), walked chunk by chunk with the oracle's locator."""
    out = []
    e = 0
    while e < count:
        ch, lp, _, first, ln = orc.locate(n, count, dtype, nch, chunk, e)
        out.append((ch, lp))
        e = first + ln
    last = {}
    for ch, lp in out:
        last[ch] = max(last.get(ch, -1), lp)
    return last


def multi_loop_count(n, nch, chunk):
    """Per channel: two full loops of n chunks, half a loop more, and a
    ragged tail that no 16-byte grain divides."""
    return nch * (5 * n * chunk // 2) + 4099


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "uint64"])
@pytest.mark.parametrize("nch", [1, 2])
def test_two_full_loops_and_a_shrunk_one(B, gu, orc, proto, dtype, nch):
    n = 8
    op = "probe" if dtype == "uint64" else "sum"
    with B.Comm(n, nch, proto) as comm:
        chunk = comm.plan(1 << 20, dtype)["chunkElems"]
        count = multi_loop_count(n, nch, chunk)
        plan, _, _ = gu.parity_case(n, count, dtype, op, proto, nch, seed=11, comm=comm)
    assert plan["chunkElems"] == chunk and plan["nChannels"] == nch
    last = loops_per_channel(orc, n, count, dtype, nch, chunk)
    assert len(last) == nch and all(lp >= 2 for lp in last.values()), last


@pytest.mark.parametrize("proto", PROTOS)
def test_multi_loop_with_ragged_lanes_and_in_place(B, gu, orc, proto):
    # three lanes split each chunk unevenly; in place reads chunk c before
    # writing it, loop after loop
    n, nch = 8, 2
    with B.Comm(n, nch, proto) as comm:
        chunk = comm.plan(1 << 20, "float32")["chunkElems"]
        count = multi_loop_count(n, nch, chunk)
        B.arSetDebug(comm.handle, B.arDebugLanes, 3)
        plan, _, _ = gu.parity_case(n, count, "float32", "sum", proto, nch, seed=12, comm=comm)
        assert plan["lanesPerChannel"] == 3
        gu.parity_case(n, count, "bfloat16", "sum", proto, nch, seed=13, comm=comm, inplace=True)


@pytest.mark.parametrize("n,proto", [(3, "simple"), (5, "ll"), (16, "ll128"), (16, "simple"), (24, "ll"),
                                     (24, "simple")])
def test_multi_loop_other_ring_lengths(B, gu, orc, n, proto):
    # odd rings, a full 16-member workgroup, and a ring cut into workgroups
    with B.Comm(n, 1, proto) as comm:
        chunk = comm.plan(1 << 20, "float32")["chunkElems"]
        count = multi_loop_count(n, 1, chunk)
        gu.parity_case(n, count, "float32", "sum", proto, 1, seed=n, comm=comm)


@pytest.mark.parametrize("proto", PROTOS)
def test_multi_loop_max_min_int32(B, gu, orc, proto):
    n, nch = 6, 2
    with B.Comm(n, nch, proto) as comm:
        chunk = comm.plan(1 << 20, "int32")["chunkElems"]
        count = multi_loop_count(n, nch, chunk)
        for op in ("max", "min", "sum"):
            gu.parity_case(n, count, "int32", op, proto, nch, seed=21, comm=comm)


# ---------------------------------------------------------------- the halves

@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("nch", [1, 3])
def test_reduce_scatter_blocks_of_several_chunks(B, gu, orc, proto, nch):
    from test_gpu_rs_ag import rs_case
    n = 8
    with B.Comm(n, nch, proto) as comm:
        chunk = comm.plan(1 << 20, "float32", func="reducescatter")["chunkElems"]
        # each channel's share of a block: two and a half chunks, ragged
        count = nch * (5 * chunk // 2) + 4099 // 4 * 4
        rs_case(B, gu, orc, n, count, "float32", "sum", proto, nch, seed=31, comm=comm)
        # a ragged 16-bit block (LL128 needs 128-byte blocks, so one line more there)
        rs_case(B, gu, orc, n, count + (64 if proto == "ll128" else 3), "bfloat16", "sum", proto, nch, seed=32,
                comm=comm)


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("nch", [1, 3])
def test_all_gather_blocks_of_several_chunks(B, gu, orc, proto, nch):
    from test_gpu_rs_ag import ag_case
    n = 8
    with B.Comm(n, nch, proto) as comm:
        chunk = comm.plan(1 << 20, "float32", func="allgather")["chunkElems"]
        count = nch * (5 * chunk // 2) + 4096
        ag_case(B, gu, orc, n, count, "float32", proto, nch, seed=33, comm=comm)
        ag_case(B, gu, orc, n, count + (64 if proto == "ll128" else 5), "float16", proto, nch, seed=34, comm=comm)


def test_reduce_scatter_order_probe_several_chunks(B, gu, orc):
    from test_gpu_rs_ag import rs_case
    n, nch = 5, 2
    with B.Comm(n, nch, "simple") as comm:
        chunk = comm.plan(1 << 20, "uint64", func="reducescatter")["chunkElems"]
        rs_case(B, gu, orc, n, nch * (5 * chunk // 2) + 7, "uint64", "probe", "simple", nch, comm=comm)

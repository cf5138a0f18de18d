"""GPU parity of the standalone ReduceScatter and AllGather (the two halves of
the ring) against the oracle, bit for bit on every rank, through the C ABI."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

PROTOS = ["simple", "ll", "ll128"]
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


def ll128_refused(B, gu, proto, count, dtype, offset, call):
    """Forcing LL128 needs 128-byte aligned buffers and rank blocks [pages:
    LL128 alignment]; returns True (after checking the refusal) when they are not."""
    if proto != "ll128" or (count * gu.ELEM[dtype]) % 128 == 0 and offset == 0:
        return False
    with pytest.raises(B.ArError) as e:
        call()
    assert e.value.code == B.arInvalidUsage
    return True


def rs_case(B, gu, orc, n, count, dtype, op, proto, nch, seed=0, inplace=False, offset=0, comm=None):
    from ring_allreduce_reduction_amd import inputs as gen
    gu.note("reduce-scatter n=%d count=%d %s %s %s nch=%d inplace=%s offset=%d"
            % (n, count, dtype, op, proto, nch, inplace, offset))
    xs = gen.probe_inputs(n, n * count) if op == "probe" else gen.make_inputs(n, n * count, dtype, seed=seed)
    own = comm is None
    if own:
        comm = B.Comm(n, nch, proto)
    else:
        comm.set_config(proto, nch)
    try:
        sends = [gu.to_device(x, dtype, offset_elems=offset) for x in xs]
        if inplace:
            recvs = [sends[r][r * count:(r + 1) * count] for r in range(n)]
        else:
            recvs = [gu.empty_like_sentinel(count, dtype, offset_elems=offset) for _ in range(n)]
        call = lambda: comm.reduce_scatter(sends, recvs, op, recvcount=count, dtype=B.DTYPE_BY_NAME[dtype])
        if ll128_refused(B, gu, proto, count, dtype, offset, call):
            return xs, None
        call()
        torch.cuda.synchronize()
        assert comm.async_error() == B.arSuccess
        want = orc.reduce_scatter(xs, dtype, op)
        for r in range(n):
            gu.assert_bits_equal(gu.to_host_raw(recvs[r], dtype), want[r], dtype, "RS rank %d" % r)
        return xs, want
    finally:
        if own:
            comm.close()


def ag_case(B, gu, orc, n, count, dtype, proto, nch, seed=0, inplace=False, offset=0, comm=None):
    from ring_allreduce_reduction_amd import inputs as gen
    gu.note("all-gather n=%d count=%d %s %s nch=%d inplace=%s offset=%d" % (n, count, dtype, proto, nch, inplace,
                                                                           offset))
    xs = gen.make_inputs(n, count, dtype, seed=seed)
    own = comm is None
    if own:
        comm = B.Comm(n, nch, proto)
    else:
        comm.set_config(proto, nch)
    try:
        recvs = [gu.empty_like_sentinel(n * count, dtype, offset_elems=offset) for _ in range(n)]
        if inplace:
            sends = []
            for r in range(n):
                view = recvs[r][r * count:(r + 1) * count]
                view.copy_(gu.to_device(xs[r], dtype))
                sends.append(view)
        else:
            sends = [gu.to_device(x, dtype, offset_elems=offset) for x in xs]
        call = lambda: comm.all_gather(sends, recvs, sendcount=count, dtype=B.DTYPE_BY_NAME[dtype])
        if ll128_refused(B, gu, proto, count, dtype, offset, call):
            return
        call()
        torch.cuda.synchronize()
        assert comm.async_error() == B.arSuccess
        want = orc.all_gather(xs, dtype)
        for r in range(n):
            gu.assert_bits_equal(gu.to_host_raw(recvs[r], dtype), want[r], dtype, "AG rank %d" % r)
    finally:
        if own:
            comm.close()


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("dtype", ["int32", "float32", "float16", "bfloat16"])
@pytest.mark.parametrize("op", ["sum", "max", "min"])
def test_reduce_scatter_dtype_op(B, gu, orc, proto, dtype, op):
    rs_case(B, gu, orc, 6, 20480, dtype, op, proto, 4, seed=7)
    rs_case(B, gu, orc, 6, 20011, dtype, op, proto, 4, seed=8)     # ragged blocks


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("n,count,nch", [(2, 1, 1), (2, 4099, 2), (3, 777, 3), (8, 65536, 16), (8, 100003, 5),
                                         (16, 12345, 4), (16, 8192, 4), (24, 5000, 3), (24, 4096, 5)])
def test_reduce_scatter_shapes(B, gu, orc, proto, n, count, nch):
    rs_case(B, gu, orc, n, count, "float32", "sum", proto, nch, seed=n + count)


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("n", [2, 5, 13])
def test_reduce_scatter_order_probe(B, gu, orc, proto, n):
    rs_case(B, gu, orc, n, 1001, "uint64", "probe", proto, 2)


@pytest.mark.parametrize("proto", ["simple", "ll"])
def test_reduce_scatter_in_place_and_unaligned(B, gu, orc, proto):
    rs_case(B, gu, orc, 8, 30000, "float32", "sum", proto, 4, inplace=True)
    rs_case(B, gu, orc, 8, 30001, "bfloat16", "sum", proto, 4, inplace=True)
    rs_case(B, gu, orc, 4, 30011, "float32", "sum", proto, 3, offset=1)      # blocks not 16-byte aligned


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("dtype", ["int32", "float32", "bfloat16"])
@pytest.mark.parametrize("n,count,nch", [(2, 1, 1), (3, 777, 2), (8, 100003, 5), (8, 131072, 8), (16, 12345, 4),
                                         (24, 5001, 3), (24, 4096, 3)])
def test_all_gather(B, gu, orc, proto, dtype, n, count, nch):
    ag_case(B, gu, orc, n, count, dtype, proto, nch, seed=n)


@pytest.mark.parametrize("direct", [0, 1])
@pytest.mark.parametrize("slot", [1, 8])
def test_all_gather_simple_variants(B, gu, orc, direct, slot):
    with B.Comm(8, 16, "simple") as comm:
        B.arSetDebug(comm.handle, B.arDebugDirect, direct)
        B.arSetDebug(comm.handle, B.arDebugSimpleSlotKiB, slot)
        ag_case(B, gu, orc, 8, 262147, "float32", "simple", 16, comm=comm)
        ag_case(B, gu, orc, 8, 70001, "float16", "simple", 3, comm=comm, inplace=True)
        rs_case(B, gu, orc, 8, 262147, "float32", "sum", "simple", 16, comm=comm)


@pytest.mark.parametrize("proto", PROTOS)
def test_rs_ag_workgroups_running_several_lanes(B, gu, orc, proto):
    with B.Comm(8, 16, proto) as comm:
        B.arSetDebug(comm.handle, B.arDebugLaneSets, 3)
        ag_case(B, gu, orc, 8, 262147, "float32", proto, 16, comm=comm)
        rs_case(B, gu, orc, 8, 262147, "float32", "sum", proto, 16, comm=comm)
        rs_case(B, gu, orc, 8, 30001, "bfloat16", "max", proto, 4, comm=comm)


def test_all_gather_unaligned(B, gu, orc):
    ag_case(B, gu, orc, 4, 30011, "float32", "simple", 3, offset=1)
    ag_case(B, gu, orc, 4, 3001, "bfloat16", "ll", 3, offset=1)


def test_allreduce_equals_allgather_of_reducescatter(B, gu, orc):
    # exact for integers [the pages: AllReduce = ReduceScatter + AllGather]
    from ring_allreduce_reduction_amd import inputs as gen
    n, count = 8, 50000
    xs = gen.make_inputs(n, n * count, "int32", seed=11)
    with B.Comm(n, 8, "simple") as comm:
        sends = [gu.to_device(x, "int32") for x in xs]
        mids = [gu.empty_like_sentinel(count, "int32") for _ in range(n)]
        outs = [gu.empty_like_sentinel(n * count, "int32") for _ in range(n)]
        ars = [gu.empty_like_sentinel(n * count, "int32") for _ in range(n)]
        comm.reduce_scatter(sends, mids, "sum")
        comm.all_gather(mids, outs)
        comm.allreduce(sends, ars, "sum")
        torch.cuda.synchronize()
        assert comm.async_error() == B.arSuccess
        for r in range(n):
            assert torch.equal(outs[r], ars[r])


def test_rs_ag_argument_checks(B, gu):
    import ctypes
    with B.Comm(4, 2, "simple") as comm:
        L = B.lib()
        big = [torch.zeros(4 * 64, device="cuda") for _ in range(4)]
        small = [torch.zeros(64, device="cuda") for _ in range(4)]
        # ReduceScatter output placed at the wrong block of its input: refused
        bad = B._ptrs([big[r][((r + 1) % 4) * 64:].data_ptr() for r in range(4)])
        assert L.arReduceScatter(comm.handle, B._ptrs(big), bad, 64, 1, 0, None) == B.arInvalidArgument
        # AllGather input overlapping another rank's output: refused
        cross = B._ptrs([big[(r + 1) % 4].data_ptr() for r in range(4)])
        assert L.arAllGather(comm.handle, cross, B._ptrs(big), 64, 1, None) == B.arInvalidArgument
        assert L.arAllGather(comm.handle, B._ptrs(small), B._ptrs(big), 64, 9, None) == B.arInvalidArgument
        assert L.arReduceScatter(comm.handle, B._ptrs(big), B._ptrs(small), 0, 1, 0, None) == B.arSuccess
        nul = (ctypes.c_void_p * 4)(0, 0, 0, 0)
        assert L.arAllGather(comm.handle, nul, B._ptrs(big), 64, 1, None) == B.arInvalidArgument


@pytest.mark.parametrize("coll", ["reducescatter", "allgather"])
def test_full_size_8_ranks_fp32(B, gu, orc, coll):
    # 8 ranks, 32 MiB blocks (256 MiB per rank on the big side), Simple 64 ch
    from ring_allreduce_reduction_amd import inputs as gen
    n, count = 8, 8 * MiB
    if coll == "reducescatter":
        xs = gen.make_inputs(n, n * count, "float32", seed=0)
        with B.Comm(n, 64, "auto") as comm:
            gu.note("reduce-scatter 8 x 256 MiB fp32 auto")
            sends = [gu.to_device(x, "float32") for x in xs]
            recvs = [gu.empty_like_sentinel(count, "float32") for _ in range(n)]
            comm.reduce_scatter(sends, recvs, "sum")
            torch.cuda.synchronize()
            assert comm.async_error() == B.arSuccess
            want = orc.reduce_scatter(xs, "float32", "sum")
            for r in range(n):
                gu.assert_bits_equal(gu.to_host_raw(recvs[r], "float32"), want[r], "float32", "RS rank %d" % r)
    else:
        xs = gen.make_inputs(n, count, "float32", seed=0)
        with B.Comm(n, 64, "auto") as comm:
            gu.note("all-gather 8 x 32 MiB fp32 auto")
            sends = [gu.to_device(x, "float32") for x in xs]
            recvs = [gu.empty_like_sentinel(n * count, "float32") for _ in range(n)]
            comm.all_gather(sends, recvs)
            torch.cuda.synchronize()
            assert comm.async_error() == B.arSuccess
            ref = torch.cat(sends)
            for r in range(n):
                assert torch.equal(recvs[r], ref)

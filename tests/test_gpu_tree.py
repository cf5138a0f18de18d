"""GPU parity of the double-binary-tree AllReduce against the oracle's tree
fold, bit for bit on every rank, through the C ABI."""
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


def tree(gu, n, count, dtype, op, proto, nch, **kw):
    plan, want, xs = gu.parity_case(n, count, dtype, op, proto, nch, algo="tree", **kw)
    assert plan["algo"] == 1 or n == 1
    return plan, want, xs


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("dtype", ["int32", "float32", "float16", "bfloat16"])
@pytest.mark.parametrize("op", ["sum", "max", "min"])
def test_tree_dtype_op(B, gu, proto, dtype, op):
    tree(gu, 6, 20480, dtype, op, proto, 4, seed=7)
    tree(gu, 6, 20011, dtype, op, proto, 3, seed=8)      # ragged lane shares


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("n,count,nch", [(2, 1, 1), (2, 4099, 2), (3, 777, 3), (5, 100003, 5), (7, 1, 2),
                                         (8, 65536, 16), (8, 262147, 64), (13, 12345, 4), (16, 8192, 4),
                                         (17, 3001, 2), (24, 5000, 3), (72, 20000, 8)])
def test_tree_shapes(B, gu, proto, n, count, nch):
    tree(gu, n, count, "float32", "sum", proto, nch, seed=n + count)


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("n", [2, 4, 5, 8, 13, 24])
def test_tree_order_probe(B, gu, proto, n):
    tree(gu, n, 1001, "uint64", "probe", proto, 2)


@pytest.mark.parametrize("proto", ["simple", "ll"])
def test_tree_in_place_and_unaligned(B, gu, proto):
    tree(gu, 8, 30000, "float32", "sum", proto, 4, inplace=True)
    tree(gu, 8, 30001, "bfloat16", "sum", proto, 4, inplace=True)
    tree(gu, 4, 30011, "float32", "sum", proto, 3, offset=1)


@pytest.mark.parametrize("slots", [2, 8])
@pytest.mark.parametrize("lanes", [1, 3])
def test_tree_many_columns_per_lane(B, gu, slots, lanes):
    # few lanes, shallow FIFOs: every lane share runs many batches of columns
    with B.Comm(8, 4, "simple", "tree") as comm:
        B.arSetDebug(comm.handle, B.arDebugSlots, slots)
        B.arSetDebug(comm.handle, B.arDebugLanes, lanes)
        for proto in PROTOS:
            gu.parity_case(8, 200003, "float32", "sum", proto, 4, comm=comm)


def test_tree_8x64MiB_fp32_full(B, gu, orc):
    tree(gu, 8, 16 << 20, "float32", "sum", "simple", 16, seed=0)


def test_ring_and_tree_share_a_comm(B, gu):
    # counters and LL flags stay consistent when one comm alternates algorithms
    with B.Comm(8, 4, "ll", "ring") as comm:
        for i, algo in enumerate(["ring", "tree", "ring", "tree", "tree", "ring"]):
            comm.set_algo(algo)
            for proto in PROTOS:
                plan, _, _ = gu.parity_case(8, 10007 + i, "float32", "sum", proto, 4, comm=comm, seed=i)
                assert B.ALGO_NAMES[plan["algo"]] == algo


def test_tree_comm_runs_ring_halves(B, gu, orc):
    from ring_allreduce_reduction_amd import inputs as gen
    n, count = 8, 5000
    xs = gen.make_inputs(n, n * count, "float32", seed=3)
    with B.Comm(n, 4, "simple", "tree") as comm:
        assert comm.plan(count, "float32", func="reducescatter")["algo"] == B.arAlgoRing
        sends = [gu.to_device(x, "float32") for x in xs]
        recvs = [gu.empty_like_sentinel(count, "float32") for _ in range(n)]
        comm.reduce_scatter(sends, recvs, "sum")
        torch.cuda.synchronize()
        want = orc.reduce_scatter(xs, "float32", "sum")
        for r in range(n):
            gu.assert_bits_equal(gu.to_host_raw(recvs[r], "float32"), want[r], "float32", "RS rank %d" % r)


def test_tree_equals_ring_on_integers(B, gu):
    from ring_allreduce_reduction_amd import inputs as gen
    n, count = 8, 70001
    xs = gen.make_inputs(n, count, "int32", seed=12)
    outs = {}
    for algo in ("ring", "tree"):
        _, want, _ = gu.parity_case(n, count, "int32", "sum", "simple", 8, inputs=xs, algo=algo)
        outs[algo] = want
    assert np.array_equal(outs["ring"], outs["tree"])


@pytest.mark.parametrize("log2_bytes", [3, 10, 14, 17, 20, 23, 26])
def test_auto_algorithm(B, gu, log2_bytes):
    n, count = 8, (1 << log2_bytes) // 4
    with B.Comm(n, 64, "auto", "auto") as comm:
        plan, _, _ = gu.parity_case(n, count, "float32", "sum", "auto", 64, comm=comm, seed=log2_bytes)
        gu.note("auto %d B -> %s %s nch=%d" % (count * 4, B.ALGO_NAMES[plan["algo"]], B.PROTO_NAMES[plan["proto"]],
                                                plan["nChannels"]))


def test_tree_one_rank_and_empty(B, gu):
    gu.parity_case(1, 1000, "float32", "sum", "simple", 2, algo="tree")
    with B.Comm(4, 2, "simple", "tree") as comm:
        x = [torch.zeros(8, device="cuda") for _ in range(4)]
        comm.allreduce(x, x, "sum", count=0, dtype=B.arFloat32)
        torch.cuda.synchronize()
        assert comm.async_error() == B.arSuccess


@pytest.mark.parametrize("n", [2, 3, 5, 8, 16, 40, 72])
def test_tuner_follows_the_table_with_model_channels(B, n):
    # a comm takes the candidate with the shortest time in the tuner's table
    # (ring Simple, LL128, LL, then tree on ties), at the channel count the
    # cost model gives that candidate with its caps scaled for N ranks on one
    # HBM (ring x 8/N, tree x 44/(6N-4))
    f32 = np.float32
    order = [(0, 2), (0, 1), (0, 0), (1, 2), (1, 1), (1, 0)]
    with B.Comm(n, 64, "auto", "auto") as comm:
        ring = [B.arTuneGetAlgoModel(comm.handle, B.arAlgoRing, p) for p in range(3)]
        tree = [B.arTuneGetAlgoModel(comm.handle, B.arAlgoTree, p) for p in range(3)]
        ring_s = [m[:3] + (float(f32(m[3]) * (f32(8) / f32(n))),) for m in ring]
        tree_s = [m[:3] + (float(f32(m[3]) * (f32(44) / f32(6 * n - 4))),) for m in tree]
        for log2_bytes in (3, 12, 17, 20, 22, 23, 24, 26, 28):
            nbytes = 1 << log2_bytes
            a, p, ch, t = B.arTuneAlgo(comm.handle, nbytes)
            times = [(B.arTuneTableTime(n, nbytes, al, pr), i) for i, (al, pr) in enumerate(order)]
            best, bi = min((tt, i) for tt, i in times if tt is not None)
            assert (a, p) == order[bi] and t == pytest.approx(best, rel=1e-6)
            _, _, ech, _ = B.arTuneEvalAlgo(0, n, 64, nbytes, ring_s, tree_s, algoMask=1 << a, protoMask=1 << p)
            assert ch == ech
            if n == 16 and log2_bytes in (22, 23):
                assert a == B.arAlgoRing   # 16 ranks x 4-8 MiB: the ring is measured 1.4-1.5x faster
            if n == 3 and log2_bytes == 22:
                assert a == B.arAlgoRing   # 3 ranks x 4 MiB: the ring (FIFOs in LDS) is measured 13% faster
            if n == 8 and log2_bytes == 17:
                assert a == B.arAlgoTree   # 8 ranks x 128 KiB: the tree is measured 1.5x faster


def test_tune_file_models_reach_a_comm(B):
    """AR_TUNE_FILE's "model" lines replace the cost model's constants of
    every comm (checked in a child process: the file is read once per process)."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    path = os.path.join(os.environ.get("TMPDIR", "/tmp"), "ar_tune_models_%d.txt" % os.getpid())
    with open(path, "w") as f:
        f.write("8 4096 1 2 3 4 5 6\nmodel tree ll128 1.5 2.5 30 40\n")
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from ring_allreduce_reduction_amd import binding as B\n"
            "with B.Comm(8, 4, 'auto', 'auto') as c:\n"
            "    print(B.arTuneGetAlgoModel(c.handle, B.arAlgoTree, B.arProtoLL128))\n"
            "    print(B.arTuneAlgo(c.handle, 4096))\n" % root)
    try:
        r = subprocess.run([sys.executable, "-c", code], env=dict(os.environ, AR_TUNE_FILE=path),
                           capture_output=True, text=True, timeout=300)
    finally:
        os.remove(path)
    assert r.returncode == 0, r.stderr
    lines = r.stdout.strip().splitlines()
    assert lines[0] == str((1.5, 2.5, 30.0, 40.0))
    assert lines[1].startswith("(0, 0, 1,")   # the file's table: ring LL is the fastest there


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("n,count", [(72, 1 << 20), (48, 1 << 20), (24, 3 << 18)])
def test_grouped_tree_channels_for_bytes_in_flight(B, gu, proto, n, count):
    # past 16 ranks a single-call tree may run a power-of-two fraction of the
    # channels asked for, with more lanes; the result is that of the count run
    plan, _, _ = tree(gu, n, count, "float32", "sum", proto, 64, seed=n)
    nch = plan["nChannels"]
    assert 1 <= nch <= 64 and 64 % nch == 0 and plan["ranksPerGroup"] <= 16
    gu.note("tree n=%d %d B %s: %d ch x %d lanes, %d B slots, groups of %d"
            % (n, count * 4, proto, nch, plan["lanesPerChannel"], plan["stepBytes"], plan["ranksPerGroup"]))

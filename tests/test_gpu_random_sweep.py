"""Seeded randomized parity sweep on the GPU.

Cases are drawn from one seeded generator: ring length 2-24, collective
(AllReduce on the ring or the double tree, ReduceScatter, AllGather),
protocol, element type and op, channel count, and a size class -- a few
elements, part of one loop, or several loops of the protocol's chunk per
channel with a ragged tail -- plus in-place and unaligned buffers.  Every
case checks the pages' definition of the result, that each rank ends with
the same full reduction ["NCCL 原始碼解讀：一個 AllReduce 的 GPU 旅程", ch.1
§1.3], bit for bit against the oracle run on the plan that ran.  Run it with
pytest -x: it stops at the first case that differs, and the case's
parameters are printed before it runs.

A second draw widens the plans: rings and trees of up to 72 ranks (cut into
workgroups past 16, or below that by a group-size cap), the automatic
algorithm and protocol, and the plan knobs a caller can force (FIFO slots in
LDS or device memory, Simple slot size, FIFO depth, lanes per channel)."""
import numpy as np
import pytest
import torch

SEED = 20261202
NCASES = 72
CHUNK_BYTES = {"simple": 1 << 20, "ll": 64 << 10, "ll128": 240 << 10}   # the library's nominal chunks
ESZ = {"int32": 4, "float32": 4, "float16": 2, "bfloat16": 2, "uint64": 8}
MAX_RANK_BYTES = 24 << 20


def draw_cases(seed=SEED, ncases=NCASES):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(ncases):
        n = int(rng.choice([2, 3, 4, 5, 6, 7, 8, 9, 11, 12, 15, 16, 17, 20, 24]))
        func = str(rng.choice(["allreduce"] * 5 + ["tree"] * 2 + ["reducescatter", "allgather"]))
        proto = str(rng.choice(["simple", "ll", "ll128"]))
        dtype = str(rng.choice(["float32", "float32", "bfloat16", "float16", "int32", "uint64"]))
        if func == "tree" and dtype == "uint64":
            dtype = "float32"
        op = "probe" if dtype == "uint64" else str(rng.choice(["sum", "sum", "max", "min"]))
        if func == "allgather":      # no arithmetic: any element size, the probe's inputs aside
            op = "sum"
            if dtype == "uint64":
                dtype = "int32"
        nch = int(rng.integers(1, 17))
        esz = ESZ[dtype]
        chunk = CHUNK_BYTES[proto] // esz
        size_class = int(rng.integers(0, 3))
        if size_class == 0:                      # a few elements
            per = int(rng.integers(1, 400))
        elif size_class == 1:                    # part of one loop per channel
            per = int(rng.integers(400, max(401, n * chunk)))
        else:                                    # several loops per channel, ragged
            per = int(rng.uniform(1.0, 3.3) * n * chunk) + int(rng.integers(1, 4099))
        count = per if size_class == 0 else nch * per
        blocks = n if func in ("reducescatter", "allgather") else 1
        while count * blocks * esz > MAX_RANK_BYTES and count > 1:
            count //= 2
        if proto == "ll128" and blocks > 1:      # forced LL128 needs 128-byte rank blocks
            line = 128 // esz
            count = max(line, count // line * line)
        inplace = bool(rng.random() < 0.2)
        offset = 1 if (rng.random() < 0.15 and proto != "ll128") else 0
        cases.append(dict(idx=i, n=n, func=func, proto=proto, dtype=dtype, op=op, nch=nch, count=count,
                          inplace=inplace, offset=offset))
    return cases


CASES = draw_cases()


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


def test_cases_cover_every_branch():
    """The draw reaches every collective, protocol, element type and size
    class, multi-loop channels, rings cut into workgroups, in place and
    unaligned buffers (checked on the host, no GPU needed)."""
    cs = CASES
    assert {c["func"] for c in cs} == {"allreduce", "tree", "reducescatter", "allgather"}
    assert {c["proto"] for c in cs} == {"simple", "ll", "ll128"}
    assert {c["dtype"] for c in cs} == set(ESZ)
    assert any(c["n"] > 16 for c in cs) and any(c["n"] % 2 == 1 for c in cs)
    assert any(c["inplace"] for c in cs) and any(c["offset"] for c in cs)
    multi = [c for c in cs if c["func"] == "allreduce"
             and c["count"] // c["nch"] >= 2 * c["n"] * CHUNK_BYTES[c["proto"]] // ESZ[c["dtype"]]]
    assert len(multi) >= 3, "too few AllReduce cases with two full loops per channel"


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=["case%02d" % c["idx"] for c in CASES])
def test_random_case(B, gu, orc, case):
    c = case
    n, count, dtype, op, proto, nch = c["n"], c["count"], c["dtype"], c["op"], c["proto"], c["nch"]
    if c["func"] in ("allreduce", "tree"):
        gu.parity_case(n, count, dtype, op, proto, nch, seed=SEED + c["idx"], inplace=c["inplace"],
                       offset=c["offset"], algo="tree" if c["func"] == "tree" else "ring")
    elif c["func"] == "reducescatter":
        from test_gpu_rs_ag import rs_case
        rs_case(B, gu, orc, n, count, dtype, op, proto, nch, seed=SEED + c["idx"], inplace=c["inplace"],
                offset=c["offset"])
    else:
        from test_gpu_rs_ag import ag_case
        ag_case(B, gu, orc, n, count, dtype, proto, nch, seed=SEED + c["idx"], inplace=c["inplace"],
                offset=c["offset"])


WIDE_SEED = 20261203
WIDE_NCASES = 48


def draw_wide_cases(seed=WIDE_SEED, ncases=WIDE_NCASES):
    """Sizes log-uniform from one element to 8 MiB per rank; knobs as
    (name, value) pairs applied with arSetDebug before the call."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(ncases):
        n = int(rng.choice([2, 3, 5, 8, 13, 16, 17, 19, 24, 31, 32, 40, 48, 57, 64, 72]))
        func = str(rng.choice(["allreduce"] * 5 + ["reducescatter", "allgather"]))
        algo = str(rng.choice(["ring", "ring", "tree", "auto"])) if func == "allreduce" else "ring"
        proto = str(rng.choice(["simple", "simple", "ll", "ll128", "auto"]))
        if func != "allreduce" and proto == "auto":
            proto = "simple"
        dtype = str(rng.choice(["float32", "float32", "bfloat16", "float16", "int32", "uint64"]))
        if algo != "ring" and dtype == "uint64":
            dtype = "float32"
        op = "probe" if dtype == "uint64" else str(rng.choice(["sum", "sum", "max", "min"]))
        if func == "allgather":
            op = "sum"
            if dtype == "uint64":
                dtype = "int32"
        nch = int(rng.choice([1, 2, 3, 4, 7, 8, 16, 32, 64]))
        esz = ESZ[dtype]
        count = max(1, int(2 ** rng.uniform(0, 23)) // esz + int(rng.integers(0, 5)))
        blocks = n if func != "allreduce" else 1
        while count * blocks * esz * n > (1 << 30) and count > 1:
            count //= 2
        if proto == "ll128" and blocks > 1:
            line = 128 // esz
            count = max(line, count // line * line)
        inplace = bool(rng.random() < 0.2)
        offset = 1 if (rng.random() < 0.15 and proto not in ("ll128", "auto")) else 0
        knobs = []
        if rng.random() < 0.3:
            knobs.append(("arDebugLdsFifo", int(rng.integers(0, 2))))
        if rng.random() < 0.2:
            knobs.append(("arDebugSimpleSlotKiB", int(rng.choice([1, 2, 4, 8]))))
        if rng.random() < 0.2:
            knobs.append(("arDebugSlots", int(rng.integers(2, 9))))
        if rng.random() < 0.2 and n > 2:
            knobs.append(("arDebugGroupSize", int(rng.choice([2, 3, 4, 6, 8, 9, 12, 16]))))
        if rng.random() < 0.15:
            knobs.append(("arDebugLanes", int(rng.choice([1, 2, 4]))))
        cases.append(dict(idx=i, n=n, func=func, algo=algo, proto=proto, dtype=dtype, op=op, nch=nch,
                          count=count, inplace=inplace, offset=offset, knobs=knobs))
    return cases


WIDE_CASES = draw_wide_cases()


def test_wide_cases_cover_every_branch():
    """The wide draw reaches rings and trees cut into workgroups, both FIFO
    placements, every forced knob, and the automatic algorithm and protocol
    (checked on the host)."""
    cs = WIDE_CASES
    assert any(c["n"] > 16 and c["func"] == "allreduce" and c["algo"] == "ring" for c in cs)
    assert any(c["n"] > 16 and c["algo"] == "tree" for c in cs)
    assert {c["algo"] for c in cs} == {"ring", "tree", "auto"}
    assert "auto" in {c["proto"] for c in cs}
    forced = {k for c in cs for k, _ in c["knobs"]}
    assert forced == {"arDebugLdsFifo", "arDebugSimpleSlotKiB", "arDebugSlots", "arDebugGroupSize",
                      "arDebugLanes"}
    assert {v for c in cs for k, v in c["knobs"] if k == "arDebugLdsFifo"} == {0, 1}


@pytest.mark.gpu
@pytest.mark.parametrize("case", WIDE_CASES, ids=["wide%02d" % c["idx"] for c in WIDE_CASES])
def test_random_wide_case(B, gu, orc, case):
    c = case
    n, count, dtype, op, proto, nch = c["n"], c["count"], c["dtype"], c["op"], c["proto"], c["nch"]
    gu.note("wide case %d: %s algo=%s knobs=%s" % (c["idx"], c["func"], c["algo"], c["knobs"]))
    comm = B.Comm(n, nch, proto, c["algo"])
    try:
        for name, value in c["knobs"]:
            B.arSetDebug(comm.handle, getattr(B, name), value)
        seed = WIDE_SEED + c["idx"]
        if c["func"] == "allreduce":
            gu.parity_case(n, count, dtype, op, proto, nch, seed=seed, inplace=c["inplace"], offset=c["offset"],
                           comm=comm)
        elif c["func"] == "reducescatter":
            from test_gpu_rs_ag import rs_case
            rs_case(B, gu, orc, n, count, dtype, op, proto, nch, seed=seed, inplace=c["inplace"],
                    offset=c["offset"], comm=comm)
        else:
            from test_gpu_rs_ag import ag_case
            ag_case(B, gu, orc, n, count, dtype, proto, nch, seed=seed, inplace=c["inplace"],
                    offset=c["offset"], comm=comm)
    finally:
        comm.close()

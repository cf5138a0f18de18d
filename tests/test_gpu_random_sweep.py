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
parameters are printed before it runs."""
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

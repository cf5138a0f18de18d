"""C-ABI checks that need no GPU: the library loads, exports every function
include/ar.h declares, rejects bad arguments before touching HIP, and the
tuner's closed forms and tie-breaks hold."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def B():
    from ring_allreduce_reduction_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from ring_allreduce_reduction_amd.build import build
        build()
    binding.lib()
    return binding


def _declared():
    src = open(os.path.join(ROOT, "include", "ar.h")).read()
    return re.findall(r"^(?:arResult_t|const char\*)\s+(ar\w+)\s*\(", src, re.M)


def test_header_declares_the_boundary():
    names = set(_declared())
    for fn in ("arInit", "arAllReduce", "arTune", "arCommGetAsyncError", "arCommAbort", "arCommCount", "arDestroy",
               "arGetErrorString", "arTuneEval", "arGetPlan", "arSetConfig", "arSetAlgo", "arTuneAlgo",
               "arTuneEvalAlgo", "arTuneGetAlgoModel", "arTuneSetAlgoModel"):
        assert fn in names


def test_every_declared_symbol_is_exported(B):
    L = ctypes.CDLL(B.LIB_PATH)
    for fn in _declared():
        assert hasattr(L, fn), fn


def test_error_strings(B):
    for code in range(8):
        s = B.arGetErrorString(code)
        assert isinstance(s, str) and len(s) > 3
    assert "unknown" in B.arGetErrorString(99)


def test_init_rejects_bad_arguments_before_hip(B):
    L = B.lib()
    h = ctypes.c_void_p()
    assert L.arInit(None, 4, 1, B.arProtoSimple, B.arAlgoRing) == B.arInvalidArgument
    for n, ch, p, a in [(0, 1, 2, 0), (129, 1, 2, 0), (4, 0, 2, 0), (4, 65, 2, 0), (4, 1, 7, 0), (4, 1, -2, 0),
                        (4, 1, 2, 2), (4, 1, 2, -2)]:
        assert L.arInit(ctypes.byref(h), n, ch, p, a) == B.arInvalidArgument, (n, ch, p, a)
        assert h.value is None


def test_init_without_gpu_reports_hip_error(B):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    L = B.lib()
    h = ctypes.c_void_p()
    assert L.arInit(ctypes.byref(h), 4, 1, B.arProtoSimple, B.arAlgoRing) == B.arHipError
    assert h.value is None


def test_calls_on_a_null_comm(B):
    L = B.lib()
    ptrs = (ctypes.c_void_p * 1)(0)
    assert L.arAllReduce(None, ptrs, ptrs, 4, B.arFloat32, B.arSum, None) == B.arInvalidArgument
    assert L.arTune(None, 1024, None, None, None) == B.arInvalidArgument
    assert L.arCommAbort(None) == B.arInvalidArgument
    assert L.arSetConfig(None, 2, 1) == B.arInvalidArgument
    assert L.arSetAlgo(None, 1) == B.arInvalidArgument
    assert L.arDestroy(None) == B.arSuccess
    e = ctypes.c_int()
    assert L.arCommGetAsyncError(None, ctypes.byref(e)) == B.arInvalidArgument
    assert L.arCommCount(None, ctypes.byref(e)) == B.arInvalidArgument
    # a pointer that is not a comm (no magic) is refused, not dereferenced as one
    junk = ctypes.create_string_buffer(4096)
    assert L.arAllReduce(ctypes.cast(junk, ctypes.c_void_p), ptrs, ptrs, 4, 1, 0, None) == B.arInvalidArgument
    assert L.arCommCount(ctypes.cast(junk, ctypes.c_void_p), ctypes.byref(e)) == B.arInvalidArgument


# ---------------------------------------------------------------- binding checks
# The library reads nranks pointers from each array and trusts the sizes, so
# the binding rejects short lists, mixed element types and short tensors
# before anything is passed on (CPU tensors stand in for device ones here:
# the checks look only at length, element type and element count).

def test_binding_rejects_wrong_buffer_lists(B):
    import torch
    four = [torch.zeros(64, dtype=torch.float32) for _ in range(4)]
    B._check_bufs(4, four, four, B.arFloat32, 64, 64)               # a valid call passes
    with pytest.raises(ValueError, match="need 4"):
        B._check_bufs(4, four[:3], four, B.arFloat32, 64, 64)
    with pytest.raises(ValueError, match="need 4"):
        B._check_bufs(4, four, four + four[:1], B.arFloat32, 64, 64)


def test_binding_rejects_mixed_or_wrong_element_types(B):
    import torch
    f32 = [torch.zeros(64, dtype=torch.float32) for _ in range(4)]
    mixed = f32[:3] + [torch.zeros(64, dtype=torch.int32)]
    with pytest.raises(ValueError, match="like the others"):
        B._check_bufs(4, f32, mixed, B.arFloat32, 64, 64)
    with pytest.raises(ValueError, match="byte elements"):
        B._check_bufs(4, f32, f32, B.arFloat16, 64, 64)
    with pytest.raises(ValueError, match="unknown dtype"):
        B._check_bufs(4, f32, f32, 9, 64, 64)


def test_binding_rejects_short_tensors(B):
    import torch
    blk = [torch.zeros(64, dtype=torch.float32) for _ in range(4)]
    big = [torch.zeros(4 * 64, dtype=torch.float32) for _ in range(4)]
    with pytest.raises(ValueError, match="holds 64 elements, the call touches 65"):
        B._check_bufs(4, blk, blk, B.arFloat32, 65, 65)
    # ReduceScatter: sends hold nranks blocks, receives one
    B._check_bufs(4, big, blk, B.arFloat32, 4 * 64, 64)
    with pytest.raises(ValueError, match="send buffer 0"):
        B._check_bufs(4, blk, blk, B.arFloat32, 4 * 64, 64)
    # AllGather: receives hold nranks blocks
    with pytest.raises(ValueError, match="receive buffer 0"):
        B._check_bufs(4, blk, blk, B.arFloat32, 64, 4 * 64)


# ---------------------------------------------------------------- tuner

def _t(model, proto, n, nch, nbytes):
    """The pages' ring model written out: busBw = bw*nch, LL x0.5, LL128 x0.92,
    capped; algBw = busBw*N/(2(N-1)); t = base + 2(N-1)*step + nBytes/(1000*algBw)."""
    base, step, bw, cap = model
    bus = bw * nch * {0: 0.5, 1: 0.92, 2: 1.0}[proto]
    bus = min(bus, cap)
    alg = bus * n / (2 * (n - 1))
    return base + 2 * (n - 1) * step + nbytes / (1000.0 * alg)


MODELS = [(5.0, 0.5, 10.0, 100.0), (6.0, 0.7, 10.0, 200.0), (9.0, 1.0, 10.0, 300.0)]


def test_single_rank_short_cut(B):
    assert B.arTuneEval(1, 16, 1 << 20, MODELS) == (B.arProtoSimple, 0, 0.0)


@pytest.mark.parametrize("nbytes", [8, 4096, 1 << 16, 1 << 20, 1 << 24, 1 << 28])
@pytest.mark.parametrize("n", [2, 8, 72])
def test_argmin_matches_closed_form(B, n, nbytes):
    p, ch, t = B.arTuneEval(n, 64, nbytes, MODELS)
    best = None
    for proto in (2, 1, 0):            # protocol ties keep the first visited
        bp = None
        c = 1
        while c <= 64:
            if c > 1 and nbytes // c < 32768:
                break
            tt = _t(MODELS[proto], proto, n, c, nbytes)
            if bp is None or tt <= bp[2] * (1 + 1e-6):   # channel ties keep more channels
                bp = (proto, c, tt)
            c *= 2
        if best is None or bp[2] < best[2] * (1 - 1e-6):
            best = bp
    assert (p, ch) == best[:2]
    assert t == pytest.approx(best[2], rel=1e-5)


def test_small_messages_pick_ll_large_pick_simple(B):
    assert B.arTuneEval(8, 64, 64, MODELS)[0] == B.arProtoLL
    assert B.arTuneEval(8, 64, 1 << 28, MODELS)[0] == B.arProtoSimple


def test_channels_keep_32k_per_channel(B):
    for nbytes in (1 << 15, 1 << 16, 3 << 16, 1 << 22):
        _, ch, _ = B.arTuneEval(8, 64, nbytes, MODELS)
        assert ch == 1 or nbytes // ch >= 32768
    assert B.arTuneEval(8, 64, 1 << 16, MODELS)[1] == 2   # more channels only help bandwidth


def test_ties_prefer_simple_then_more_channels(B):
    same = [(5.0, 0.5, 1e9, 10.0)] * 3   # capped from one channel on: every candidate ties
    p, ch, _ = B.arTuneEval(8, 64, 1 << 24, same)
    assert p == B.arProtoSimple and ch == 64
    p, ch, _ = B.arTuneEval(8, 64, 1 << 24, same, protoMask=0b011)
    assert p == B.arProtoLL128 and ch == 64
    p, ch, _ = B.arTuneEval(8, 64, 1 << 17, same)   # 128 KiB: at most 4 channels of 32 KiB
    assert ch == 4


def test_tuner_errors(B):
    with pytest.raises(B.ArError) as e:
        B.arTuneEval(8, 64, 1024, MODELS, protoMask=0)
    assert e.value.code == B.arInvalidArgument
    bad = [(1.0, 1.0, 0.0, 1.0)] * 3
    with pytest.raises(B.ArError) as e:
        B.arTuneEval(8, 64, 1024, bad)
    assert e.value.code == B.arInvalidUsage


@pytest.mark.parametrize("func", [1, 2])
@pytest.mark.parametrize("nbytes", [64, 1 << 20, 1 << 28])
def test_halves_use_n_minus_1_steps(B, func, nbytes):
    # ReduceScatter / AllGather: nSteps = N-1, algBw = busBw*N/(N-1) [ch.5 §三]
    n = 8
    p, ch, t = B.arTuneEvalColl(func, n, 64, nbytes, MODELS)
    base, step, bw, cap = MODELS[p]
    bus = min(bw * ch * {0: 0.5, 1: 0.92, 2: 1.0}[p], cap)
    assert t == pytest.approx(base + (n - 1) * step + nbytes / (1000.0 * bus * n / (n - 1)), rel=1e-5)
    assert B.arTuneEvalColl(0, n, 64, nbytes, MODELS) == B.arTuneEval(n, 64, nbytes, MODELS)
    with pytest.raises(B.ArError):
        B.arTuneEvalColl(3, n, 64, nbytes, MODELS)


# ---------------------------------------------------------------- tree model

# the pages' treeCorrectionFactor rows (LL, LL128, Simple), column i = 64 B * 2^i
CORR = [
    [1.0, 1.0, 1.0, 1.0, .9, .8, .7, .7, .7, .7, .6, .5, .4, .4, .5, .6, .7, .8, .9, 1.0, 1.0, 1.0, 1.0, 1.0],
    [1.0, 1.0, 1.0, 1.0, 1.0, .9, .8, .8, .8, .7, .6, .6, .6, .6, .6, .6, .8, .9, .9, .9, .9, 1.0, 1.0, 1.0],
    [.9, .9, .9, .9, .9, .9, .9, .8, .7, .6, .6, .5, .5, .5, .5, .6, .7, .8, .7, .7, .8, .9, .9, .9],
]


def _tree_t(model, proto, n, nch, nbytes):
    """The pages' tree model written out [ch.5 §四]: busBw = bw*nch*0.92, LL
    x1/3.8, LL128 x120/128, capped; x correction[proto][log2(nBytes>>6)];
    lat = base + 2*floor(log2 N)*step."""
    base, step, bw, cap = model
    bus = bw * nch * 0.92 * {0: 1 / 3.8, 1: 120 / 128, 2: 1.0}[proto]
    bus = min(bus, cap)
    q = nbytes >> 6
    if q > 0 and q.bit_length() - 1 < 23:
        bus *= CORR[proto][q.bit_length() - 1]
    return base + 2 * (n.bit_length() - 1) * step + nbytes / (1000.0 * bus)


TREE = [(3.0, 0.4, 12.0, 90.0), (4.0, 0.5, 12.0, 150.0), (6.0, 0.6, 12.0, 250.0)]


@pytest.mark.parametrize("nbytes", [8, 64, 4096, 1 << 16, 3 << 18, 1 << 20, 1 << 24, 1 << 28])
@pytest.mark.parametrize("n", [2, 8, 24, 72])
def test_tree_argmin_matches_closed_form(B, n, nbytes):
    a, p, ch, t = B.arTuneEvalAlgo(0, n, 64, nbytes, MODELS, TREE)
    best = None
    for algo, models, tf in ((0, MODELS, _t), (1, TREE, _tree_t)):
        for proto in (2, 1, 0):
            bp = None
            c = 1
            while c <= 64:
                if c > 1 and nbytes // c < 32768:
                    break
                tt = tf(models[proto], proto, n, c, nbytes)
                if bp is None or tt <= bp[3] * (1 + 1e-6):
                    bp = (algo, proto, c, tt)
                c *= 2
            if best is None or bp[3] < best[3] * (1 - 1e-6):
                best = bp
    assert (a, p, ch) == best[:3]
    assert t == pytest.approx(best[3], rel=1e-5)


def test_tree_only_for_allreduce_and_masks(B):
    fast_tree = [(0.0, 0.0, 1e6, 1e6)] * 3
    slow_ring = [(100.0, 10.0, 1.0, 1.0)] * 3
    assert B.arTuneEvalAlgo(0, 8, 64, 4096, slow_ring, fast_tree)[0] == B.arAlgoTree
    for func in (1, 2):   # ReduceScatter / AllGather: ring only
        assert B.arTuneEvalAlgo(func, 8, 64, 4096, slow_ring, fast_tree)[0] == B.arAlgoRing
    assert B.arTuneEvalAlgo(0, 8, 64, 4096, slow_ring, fast_tree, algoMask=1)[0] == B.arAlgoRing
    assert B.arTuneEvalAlgo(0, 8, 64, 4096, None, fast_tree, algoMask=2)[0] == B.arAlgoTree
    with pytest.raises(B.ArError):
        B.arTuneEvalAlgo(0, 8, 64, 4096, None, fast_tree, algoMask=3)
    with pytest.raises(B.ArError):
        B.arTuneEvalAlgo(0, 8, 64, 4096, slow_ring, fast_tree, algoMask=0)
    # an exact tie keeps the ring: at N = 8 both take 12 us of latency and
    # 8 GB/s (ring: cap 14 * 8/14; tree: cap 8, no correction past 512 MiB)
    ring = [(5.0, 0.5, 1e9, 14.0)] * 3
    tree = [(6.0, 1.0, 1e9, 8.0)] * 3
    r = B.arTuneEvalAlgo(0, 8, 64, 1 << 30, ring, tree, protoMask=4)
    assert r[0] == B.arAlgoRing and r[3] == pytest.approx(12 + (1 << 30) / 8000.0)
    assert B.arTuneEvalAlgo(0, 8, 64, 1 << 30, ring, tree, algoMask=2, protoMask=4)[3] == r[3]
    assert B.arTuneEvalAlgo(0, 1, 64, 1 << 20, ring, tree) == (B.arAlgoRing, B.arProtoSimple, 0, 0.0)


def test_ring_eval_unchanged_by_tree(B):
    for nbytes in (64, 1 << 20, 1 << 28):
        a, p, ch, t = B.arTuneEvalAlgo(0, 8, 64, nbytes, MODELS, None, algoMask=1)
        assert (p, ch) == B.arTuneEval(8, 64, nbytes, MODELS)[:2] and a == B.arAlgoRing


def test_library_links_roctx_for_api_ranges():
    """The API entry points carry ROCTx ranges (arInit, arAllReduce,
    arReduceScatter, arAllGather, arGroupEnd): the library links the ROCTx
    runtime and names the ranges.  CPU only (readelf and the file's bytes)."""
    import shutil
    import subprocess
    from ring_allreduce_reduction_amd import binding
    if shutil.which("readelf") is None:
        import pytest
        pytest.skip("readelf not found")
    dyn = subprocess.run(["readelf", "-d", binding.LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert "librocprofiler-sdk-roctx" in dyn
    blob = open(binding.LIB_PATH, "rb").read()
    for name in (b"arInit", b"arAllReduce", b"arReduceScatter", b"arAllGather", b"arGroupEnd"):
        assert name + b"\x00" in blob

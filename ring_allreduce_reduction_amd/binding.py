"""ctypes binding of libar.so -- argument marshalling only.

Every function here has the C ABI's name (include/ar.h) and passes plain
pointers and sizes through; all work runs in the library's HIP kernels.
PyTorch is used only for device memory and streams.  Loading fails loudly if
the library has not been built: there is no fallback path.
"""
import ctypes
import os

import torch  # noqa: F401  -- loads the HIP runtime the library must share

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libar.so")

# enums (include/ar.h)
arSuccess, arHipError, arSystemError, arInternalError = 0, 1, 2, 3
arInvalidArgument, arInvalidUsage, arRemoteError, arInProgress = 4, 5, 6, 7
arProtoAuto, arProtoLL, arProtoLL128, arProtoSimple = -1, 0, 1, 2
arAlgoAuto, arAlgoRing, arAlgoTree = -1, 0, 1
arInt32, arFloat32, arFloat16, arBfloat16, arUint64 = 0, 1, 2, 3, 4
arSum, arMax, arMin, arProbe = 0, 1, 2, 3
(arDebugTimeoutUs, arDebugDeadRank, arDebugLanes, arDebugSimpleSlotKiB, arDebugDirect, arDebugSlots,
 arDebugLaneSets, arDebugLL128SlotKiB, arDebugGroupSpread, arDebugLLChunkBytes,
 arDebugLL128ChunkBytes, arDebugCooperative, arDebugGroupSize, arDebugLdsFifo) = (
    0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13)
AR_MAX_RANKS, AR_MAX_CHANNELS = 128, 64
arFuncAllReduce, arFuncReduceScatter, arFuncAllGather = 0, 1, 2
FUNC_BY_NAME = {"allreduce": arFuncAllReduce, "reducescatter": arFuncReduceScatter,
                "allgather": arFuncAllGather}

PROTO_NAMES = {arProtoLL: "LL", arProtoLL128: "LL128", arProtoSimple: "Simple", arProtoAuto: "auto"}
PROTO_BY_NAME = {"ll": arProtoLL, "ll128": arProtoLL128, "simple": arProtoSimple, "auto": arProtoAuto}
DTYPE_BY_NAME = {"int32": arInt32, "float32": arFloat32, "float16": arFloat16,
                 "bfloat16": arBfloat16, "uint64": arUint64}
OP_BY_NAME = {"sum": arSum, "max": arMax, "min": arMin, "probe": arProbe}
ALGO_NAMES = {arAlgoRing: "ring", arAlgoTree: "tree", arAlgoAuto: "auto"}
ALGO_BY_NAME = {"ring": arAlgoRing, "tree": arAlgoTree, "auto": arAlgoAuto}


class arTuneModel_t(ctypes.Structure):
    _fields_ = [("baseLatUs", ctypes.c_float), ("stepLatUs", ctypes.c_float),
                ("bwPerChGBs", ctypes.c_float), ("maxBwGBs", ctypes.c_float)]


class arPlan_t(ctypes.Structure):
    _fields_ = [("proto", ctypes.c_int), ("nChannels", ctypes.c_int), ("chunkElems", ctypes.c_size_t),
                ("lanesPerChannel", ctypes.c_int), ("ranksPerGroup", ctypes.c_int),
                ("workgroups", ctypes.c_int), ("threadsPerGroup", ctypes.c_int),
                ("stepBytes", ctypes.c_int), ("stepPayload", ctypes.c_int), ("nSlots", ctypes.c_int),
                ("predictedUs", ctypes.c_float), ("modelBytes", ctypes.c_double), ("algo", ctypes.c_int),
                ("groupLaunch", ctypes.c_int), ("tasksInLaunch", ctypes.c_int), ("ldsFifoBytes", ctypes.c_int),
                ("deviceBytes", ctypes.c_double)]


class ArError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__("%s failed: %s (%d)" % (where, arGetErrorString(code), code))


_lib = None


def lib():
    """The loaded libar.so (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libar.so is not built (run __graft_entry__.build() or "
                              "python ring_allreduce_reduction_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        c_int, c_sz, vp, c_f = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
        L.arInit.argtypes = [ctypes.POINTER(vp), c_int, c_int, c_int, c_int]
        L.arAllReduce.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), c_sz, c_int, c_int, vp]
        L.arReduceScatter.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), c_sz, c_int, c_int, vp]
        L.arAllGather.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), c_sz, c_int, vp]
        L.arTune.argtypes = [vp, c_sz, ctypes.POINTER(c_int), ctypes.POINTER(c_int), ctypes.POINTER(c_f)]
        L.arTuneEvalColl.argtypes = [c_int, c_int, c_int, c_sz, ctypes.POINTER(arTuneModel_t), ctypes.c_uint,
                                     ctypes.POINTER(c_int), ctypes.POINTER(c_int), ctypes.POINTER(c_f)]
        L.arGetPlanColl.argtypes = [vp, c_int, c_sz, c_int, c_int, ctypes.POINTER(arPlan_t)]
        L.arTuneEval.argtypes = [c_int, c_int, c_sz, ctypes.POINTER(arTuneModel_t), ctypes.c_uint,
                                 ctypes.POINTER(c_int), ctypes.POINTER(c_int), ctypes.POINTER(c_f)]
        L.arTuneGetModel.argtypes = [vp, c_int, ctypes.POINTER(arTuneModel_t)]
        L.arTuneSetModel.argtypes = [vp, c_int, ctypes.POINTER(arTuneModel_t)]
        L.arSetConfig.argtypes = [vp, c_int, c_int]
        L.arSetAlgo.argtypes = [vp, c_int]
        L.arTuneAlgo.argtypes = [vp, c_sz, ctypes.POINTER(c_int), ctypes.POINTER(c_int), ctypes.POINTER(c_int),
                                 ctypes.POINTER(c_f)]
        L.arTuneEvalAlgo.argtypes = [c_int, c_int, c_int, c_sz, ctypes.POINTER(arTuneModel_t),
                                     ctypes.POINTER(arTuneModel_t), ctypes.c_uint, ctypes.c_uint,
                                     ctypes.POINTER(c_int), ctypes.POINTER(c_int), ctypes.POINTER(c_int),
                                     ctypes.POINTER(c_f)]
        L.arTuneGetAlgoModel.argtypes = [vp, c_int, c_int, ctypes.POINTER(arTuneModel_t)]
        L.arTuneSetAlgoModel.argtypes = [vp, c_int, c_int, ctypes.POINTER(arTuneModel_t)]
        L.arGroupStart.argtypes = []
        L.arGroupEnd.argtypes = []
        L.arGroupAggregate.argtypes = [c_int, ctypes.POINTER(c_int), ctypes.POINTER(c_sz), ctypes.POINTER(c_int),
                                       ctypes.POINTER(c_int), ctypes.POINTER(c_int), ctypes.POINTER(c_int)]
        L.arGetGroupPlan.argtypes = [vp, c_int, ctypes.POINTER(arPlan_t)]
        L.arGetPlan.argtypes = [vp, c_sz, c_int, c_int, ctypes.POINTER(arPlan_t)]
        L.arCommGetAsyncError.argtypes = [vp, ctypes.POINTER(c_int)]
        L.arCommAbort.argtypes = [vp]
        L.arCommCount.argtypes = [vp, ctypes.POINTER(c_int)]
        L.arCommFootprint.argtypes = [vp, ctypes.POINTER(c_sz)]
        L.arTuneTableTime.argtypes = [c_int, c_sz, c_int, c_int, ctypes.POINTER(c_f)]
        L.arAllReduceNoAlloc.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), c_int, c_int, c_sz, c_int, c_int, vp]
        L.arDestroy.argtypes = [vp]
        L.arSetDebug.argtypes = [vp, c_int, ctypes.c_int64]
        L.arGetErrorString.argtypes = [c_int]
        L.arGetErrorString.restype = ctypes.c_char_p
        for fn in ("arInit", "arAllReduce", "arReduceScatter", "arAllGather", "arTune", "arTuneEval",
                   "arTuneEvalColl", "arTuneGetModel", "arTuneSetModel", "arSetConfig", "arGetPlan", "arGetPlanColl",
                   "arSetAlgo", "arTuneAlgo", "arTuneEvalAlgo", "arTuneGetAlgoModel", "arTuneSetAlgoModel",
                   "arGroupStart", "arGroupEnd", "arGroupAggregate", "arGetGroupPlan",
                   "arCommGetAsyncError", "arCommAbort", "arCommCount", "arDestroy", "arSetDebug",
                   "arAllReduceNoAlloc", "arTuneTableTime", "arCommFootprint"):
            getattr(L, fn).restype = c_int
        _lib = L
    return _lib


def _check(code, where):
    if code != arSuccess:
        raise ArError(code, where)


def arGetErrorString(code):
    return lib().arGetErrorString(int(code)).decode()


def arInit(nranks, nChannels, proto=arProtoSimple, algo=arAlgoRing):
    h = ctypes.c_void_p()
    _check(lib().arInit(ctypes.byref(h), int(nranks), int(nChannels), int(proto), int(algo)), "arInit")
    return h


ELEM_SIZE = {arInt32: 4, arFloat32: 4, arFloat16: 2, arBfloat16: 2, arUint64: 8}


def _ptrs(bufs):
    out = []
    for b in bufs:
        if isinstance(b, torch.Tensor):
            if not b.is_cuda or not b.is_contiguous():
                raise ValueError("buffers must be contiguous device tensors")
            out.append(b.data_ptr())
        else:
            out.append(int(b))
    return (ctypes.c_void_p * len(out))(*out)


def _check_bufs(n, sendbufs, recvbufs, dtype, send_elems, recv_elems):
    """The checks the C side cannot make: the library reads exactly n
    pointers from each array, and a tensor shorter than what the call
    touches would be an out-of-bounds device access.  Tensors must share one
    element type of the call's element size and hold at least send_elems /
    recv_elems elements; raw addresses are the caller's responsibility."""
    if len(sendbufs) != n or len(recvbufs) != n:
        raise ValueError("need %d send and %d receive buffers, got %d and %d"
                         % (n, n, len(sendbufs), len(recvbufs)))
    esz = ELEM_SIZE.get(int(dtype))
    if esz is None:
        raise ValueError("unknown dtype %r" % (dtype,))
    first = None
    for what, bufs, need in (("send", sendbufs, send_elems), ("receive", recvbufs, recv_elems)):
        for r, b in enumerate(bufs):
            if not isinstance(b, torch.Tensor):
                continue
            if first is None:
                first = b.dtype
            if b.dtype != first:
                raise ValueError("%s buffer %d is %s, expected %s like the others" % (what, r, b.dtype, first))
            if b.element_size() != esz:
                raise ValueError("%s buffer %d has %d-byte elements, the call's dtype %d-byte ones"
                                 % (what, r, b.element_size(), esz))
            if b.numel() < need:
                raise ValueError("%s buffer %d holds %d elements, the call touches %d" % (what, r, b.numel(), need))


def _checked_ptrs(comm, sendbufs, recvbufs, dtype, send_elems, recv_elems):
    """Pointer arrays for a call on `comm`, after _check_bufs."""
    _check_bufs(arCommCount(comm), sendbufs, recvbufs, dtype, send_elems, recv_elems)
    return _ptrs(sendbufs), _ptrs(recvbufs)


def _dtype_of(t):
    m = {torch.int32: arInt32, torch.float32: arFloat32, torch.float16: arFloat16,
         torch.bfloat16: arBfloat16, torch.int64: arUint64}
    if hasattr(torch, "uint64"):
        m[torch.uint64] = arUint64
    return m[t.dtype]


def arAllReduce(comm, sendbufs, recvbufs, count=None, dtype=None, op=arSum, stream=None):
    """sendbufs / recvbufs: lists of device tensors (or raw device addresses,
    then count and dtype are required).  stream: a torch.cuda.Stream, a raw
    hipStream_t value, or None for torch's current stream."""
    if count is None:
        count = sendbufs[0].numel()
    if dtype is None:
        dtype = _dtype_of(sendbufs[0])
    if stream is None:
        stream = torch.cuda.current_stream()
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    sp, rp = _checked_ptrs(comm, sendbufs, recvbufs, dtype, count, count)
    _check(lib().arAllReduce(comm, sp, rp, int(count), int(dtype), int(op), ctypes.c_void_p(handle)), "arAllReduce")


def arAllReduceNoAlloc(sendbufs, recvbufs, nChannels, count=None, dtype=None, op=arSum, stream=None):
    """The comm-less, allocation-free AllReduce (ring, Simple, nranks =
    len(sendbufs) <= 16); same buffers and arguments as arAllReduce."""
    if count is None:
        count = sendbufs[0].numel()
    if dtype is None:
        dtype = _dtype_of(sendbufs[0])
    n = len(sendbufs)
    _check_bufs(n, sendbufs, recvbufs, dtype, count, count)
    _check(lib().arAllReduceNoAlloc(_ptrs(sendbufs), _ptrs(recvbufs), n, int(nChannels), int(count), int(dtype),
                                    int(op), ctypes.c_void_p(_stream_handle(stream))), "arAllReduceNoAlloc")


def _stream_handle(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def arReduceScatter(comm, sendbufs, recvbufs, recvcount=None, dtype=None, op=arSum, stream=None):
    """sendbufs[r]: nranks*recvcount elements; recvbufs[r]: recvcount elements."""
    if recvcount is None:
        recvcount = recvbufs[0].numel()
    if dtype is None:
        dtype = _dtype_of(sendbufs[0])
    n = arCommCount(comm)
    sp, rp = _checked_ptrs(comm, sendbufs, recvbufs, dtype, n * int(recvcount), recvcount)
    _check(lib().arReduceScatter(comm, sp, rp, int(recvcount), int(dtype), int(op),
                                 ctypes.c_void_p(_stream_handle(stream))), "arReduceScatter")


def arAllGather(comm, sendbufs, recvbufs, sendcount=None, dtype=None, stream=None):
    """sendbufs[r]: sendcount elements; recvbufs[r]: nranks*sendcount elements."""
    if sendcount is None:
        sendcount = sendbufs[0].numel()
    if dtype is None:
        dtype = _dtype_of(sendbufs[0])
    n = arCommCount(comm)
    sp, rp = _checked_ptrs(comm, sendbufs, recvbufs, dtype, sendcount, n * int(sendcount))
    _check(lib().arAllGather(comm, sp, rp, int(sendcount), int(dtype), ctypes.c_void_p(_stream_handle(stream))),
           "arAllGather")


def arTuneEvalColl(func, nranks, maxChannels, nBytes, models, protoMask=7):
    arr = (arTuneModel_t * 3)(*[arTuneModel_t(*m) for m in models])
    p, ch, t = ctypes.c_int(), ctypes.c_int(), ctypes.c_float()
    rc = lib().arTuneEvalColl(int(func), int(nranks), int(maxChannels), int(nBytes), arr, int(protoMask),
                              ctypes.byref(p), ctypes.byref(ch), ctypes.byref(t))
    _check(rc, "arTuneEvalColl")
    return p.value, ch.value, t.value


def arGetPlanColl(comm, func, count, dtype, aligned128=True):
    p = arPlan_t()
    _check(lib().arGetPlanColl(comm, int(func), int(count), int(dtype), 1 if aligned128 else 0, ctypes.byref(p)),
           "arGetPlanColl")
    return {f: getattr(p, f) for f, _ in arPlan_t._fields_}


def arTune(comm, nBytes):
    p, ch, t = ctypes.c_int(), ctypes.c_int(), ctypes.c_float()
    _check(lib().arTune(comm, int(nBytes), ctypes.byref(p), ctypes.byref(ch), ctypes.byref(t)), "arTune")
    return p.value, ch.value, t.value


def arTuneEval(nranks, maxChannels, nBytes, models, protoMask=7):
    arr = (arTuneModel_t * 3)(*[arTuneModel_t(*m) for m in models])
    p, ch, t = ctypes.c_int(), ctypes.c_int(), ctypes.c_float()
    rc = lib().arTuneEval(int(nranks), int(maxChannels), int(nBytes), arr, int(protoMask),
                          ctypes.byref(p), ctypes.byref(ch), ctypes.byref(t))
    _check(rc, "arTuneEval")
    return p.value, ch.value, t.value


def arTuneGetModel(comm, proto):
    m = arTuneModel_t()
    _check(lib().arTuneGetModel(comm, int(proto), ctypes.byref(m)), "arTuneGetModel")
    return (m.baseLatUs, m.stepLatUs, m.bwPerChGBs, m.maxBwGBs)


def arTuneSetModel(comm, proto, model):
    m = arTuneModel_t(*model)
    _check(lib().arTuneSetModel(comm, int(proto), ctypes.byref(m)), "arTuneSetModel")


def arSetConfig(comm, proto, nChannels):
    _check(lib().arSetConfig(comm, int(proto), int(nChannels)), "arSetConfig")


def arSetAlgo(comm, algo):
    _check(lib().arSetAlgo(comm, int(algo)), "arSetAlgo")


def arTuneAlgo(comm, nBytes):
    a, p, ch, t = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_float()
    _check(lib().arTuneAlgo(comm, int(nBytes), ctypes.byref(a), ctypes.byref(p), ctypes.byref(ch), ctypes.byref(t)),
           "arTuneAlgo")
    return a.value, p.value, ch.value, t.value


def arTuneEvalAlgo(func, nranks, maxChannels, nBytes, ringModels, treeModels, algoMask=3, protoMask=7):
    def arr(models):
        return None if models is None else (arTuneModel_t * 3)(*[arTuneModel_t(*m) for m in models])
    a, p, ch, t = ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_float()
    rc = lib().arTuneEvalAlgo(int(func), int(nranks), int(maxChannels), int(nBytes), arr(ringModels),
                              arr(treeModels), int(algoMask), int(protoMask), ctypes.byref(a), ctypes.byref(p),
                              ctypes.byref(ch), ctypes.byref(t))
    _check(rc, "arTuneEvalAlgo")
    return a.value, p.value, ch.value, t.value


def arTuneTableTime(nranks, nBytes, algo, proto):
    """The tuner table's time (us) of one candidate, or None where the table does not cover it."""
    t = ctypes.c_float()
    rc = lib().arTuneTableTime(int(nranks), int(nBytes), int(algo), int(proto), ctypes.byref(t))
    if rc == arInvalidUsage:
        return None
    _check(rc, "arTuneTableTime")
    return t.value


def arTuneGetAlgoModel(comm, algo, proto):
    m = arTuneModel_t()
    _check(lib().arTuneGetAlgoModel(comm, int(algo), int(proto), ctypes.byref(m)), "arTuneGetAlgoModel")
    return (m.baseLatUs, m.stepLatUs, m.bwPerChGBs, m.maxBwGBs)


def arTuneSetAlgoModel(comm, algo, proto, model):
    m = arTuneModel_t(*model)
    _check(lib().arTuneSetAlgoModel(comm, int(algo), int(proto), ctypes.byref(m)), "arTuneSetAlgoModel")


def arGetPlan(comm, count, dtype, aligned128=True):
    p = arPlan_t()
    _check(lib().arGetPlan(comm, int(count), int(dtype), 1 if aligned128 else 0, ctypes.byref(p)), "arGetPlan")
    return {f: getattr(p, f) for f, _ in arPlan_t._fields_}


def arGroupStart():
    _check(lib().arGroupStart(), "arGroupStart")


def arGroupEnd():
    _check(lib().arGroupEnd(), "arGroupEnd")


def arGroupAggregate(keys, nbytes, isolate=None):
    """(order, launchOf, nLaunches) of the aggregation rule."""
    n = len(keys)
    k = (ctypes.c_int * n)(*keys)
    b = (ctypes.c_size_t * n)(*nbytes)
    iso = None if isolate is None else (ctypes.c_int * n)(*isolate)
    order, launch_of, nl = (ctypes.c_int * n)(), (ctypes.c_int * n)(), ctypes.c_int()
    _check(lib().arGroupAggregate(n, k, b, iso, order, launch_of, ctypes.byref(nl)), "arGroupAggregate")
    return list(order), list(launch_of), nl.value


def arGetGroupPlan(comm, index):
    p = arPlan_t()
    _check(lib().arGetGroupPlan(comm, int(index), ctypes.byref(p)), "arGetGroupPlan")
    return {f: getattr(p, f) for f, _ in arPlan_t._fields_}


class Group:
    """with Group(): ... -- arGroupStart on entry, arGroupEnd on exit."""

    def __enter__(self):
        arGroupStart()
        return self

    def __exit__(self, exc_type, *exc):
        if exc_type is None:
            arGroupEnd()
        else:   # close the group without masking the original error
            try:
                arGroupEnd()
            except ArError:
                pass


def arCommGetAsyncError(comm):
    e = ctypes.c_int()
    _check(lib().arCommGetAsyncError(comm, ctypes.byref(e)), "arCommGetAsyncError")
    return e.value


def arCommCount(comm):
    n = ctypes.c_int()
    _check(lib().arCommCount(comm, ctypes.byref(n)), "arCommCount")
    return n.value


def arCommFootprint(comm):
    b = ctypes.c_size_t()
    _check(lib().arCommFootprint(comm, ctypes.byref(b)), "arCommFootprint")
    return b.value


def arCommAbort(comm):
    _check(lib().arCommAbort(comm), "arCommAbort")


def arSetDebug(comm, knob, value):
    _check(lib().arSetDebug(comm, int(knob), int(value)), "arSetDebug")


def arDestroy(comm):
    _check(lib().arDestroy(comm), "arDestroy")


class Comm:
    """Small convenience wrapper owning one communicator."""

    def __init__(self, nranks, nChannels, proto=arProtoSimple, algo=arAlgoRing):
        if isinstance(proto, str):
            proto = PROTO_BY_NAME[proto.lower()]
        if isinstance(algo, str):
            algo = ALGO_BY_NAME[algo.lower()]
        self.nranks = nranks
        self.handle = arInit(nranks, nChannels, proto, algo)

    def allreduce(self, sendbufs, recvbufs, op=arSum, stream=None, count=None, dtype=None):
        if isinstance(op, str):
            op = OP_BY_NAME[op]
        arAllReduce(self.handle, sendbufs, recvbufs, count=count, dtype=dtype, op=op, stream=stream)

    def plan(self, count, dtype, aligned128=True, func=arFuncAllReduce):
        if isinstance(dtype, str):
            dtype = DTYPE_BY_NAME[dtype]
        if isinstance(func, str):
            func = FUNC_BY_NAME[func]
        return arGetPlanColl(self.handle, func, count, dtype, aligned128)

    def reduce_scatter(self, sendbufs, recvbufs, op=arSum, stream=None, recvcount=None, dtype=None):
        if isinstance(op, str):
            op = OP_BY_NAME[op]
        arReduceScatter(self.handle, sendbufs, recvbufs, recvcount=recvcount, dtype=dtype, op=op, stream=stream)

    def all_gather(self, sendbufs, recvbufs, stream=None, sendcount=None, dtype=None):
        arAllGather(self.handle, sendbufs, recvbufs, sendcount=sendcount, dtype=dtype, stream=stream)

    def set_config(self, proto, nChannels):
        if isinstance(proto, str):
            proto = PROTO_BY_NAME[proto.lower()]
        arSetConfig(self.handle, proto, nChannels)

    def set_algo(self, algo):
        if isinstance(algo, str):
            algo = ALGO_BY_NAME[algo.lower()]
        arSetAlgo(self.handle, algo)

    def tune(self, nBytes):
        return arTune(self.handle, nBytes)

    def tune_algo(self, nBytes):
        return arTuneAlgo(self.handle, nBytes)

    def group_plan(self, index):
        return arGetGroupPlan(self.handle, index)

    def footprint(self):
        return arCommFootprint(self.handle)

    def async_error(self):
        return arCommGetAsyncError(self.handle)

    def close(self):
        if self.handle is not None:
            arDestroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

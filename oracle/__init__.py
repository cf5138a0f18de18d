"""CPU oracle for the ring AllReduce -- TEST INFRASTRUCTURE ONLY.

Only tests/, the package's smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library: the fold lives in
ring_oracle.c (plain single-threaded C); this file only marshals numpy arrays.

Functions mirror what the pages define (see ring_oracle.c for citations):
  allreduce()  -- the order-matched ring fold over every element
  reduce_scatter(), all_gather() -- the two halves of the ring on their own
  elements()   -- the same fold for a list of single elements
  locate()     -- channel / loop / chunk of one element
  btree(), dtree(), tree_of_channel() -- the pages' binary and double trees
  tree_allreduce(), tree_elements() -- the double-tree AllReduce fold
  direct_sum_f64(), within_tolerance() -- the float64 direct sum and the
                  error bounds the order-matched result must also meet
Pinned by tests/test_oracle_*.py (worked example, brute force, order probe,
closed forms, conversion pins against numpy and torch).
"""
import ctypes
import os

import numpy as np

from .build import LIB, build

DTYPES = {"int32": 0, "float32": 1, "float16": 2, "bfloat16": 3, "uint64": 4}
OPS = {"sum": 0, "max": 1, "min": 2, "probe": 3}
# numpy storage type per dtype (16-bit floats are carried as raw uint16 bits)
NP_STORAGE = {"int32": np.int32, "float32": np.float32, "float16": np.uint16,
              "bfloat16": np.uint16, "uint64": np.uint64}
ELEM_SIZE = {"int32": 4, "float32": 4, "float16": 2, "bfloat16": 2, "uint64": 8}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        sz, vp, i = ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int
        L.ar_oracle_allreduce.argtypes = [i, sz, i, i, i, sz, ctypes.POINTER(vp), ctypes.POINTER(vp)]
        L.ar_oracle_elements.argtypes = [i, sz, i, i, i, sz, ctypes.POINTER(vp), vp, sz, vp]
        L.ar_oracle_locate.argtypes = [i, sz, i, i, sz, sz, ctypes.POINTER(i),
                                       ctypes.POINTER(ctypes.c_longlong), ctypes.POINTER(i),
                                       ctypes.POINTER(sz), ctypes.POINTER(sz)]
        L.ar_oracle_reduce_scatter.argtypes = [i, sz, i, i, ctypes.POINTER(vp), ctypes.POINTER(vp)]
        L.ar_oracle_all_gather.argtypes = [i, sz, sz, ctypes.POINTER(vp), ctypes.POINTER(vp)]
        L.ar_oracle_btree.argtypes = [i, i] + [ctypes.POINTER(i)] * 4
        L.ar_oracle_dtree.argtypes = [i, i, i] + [ctypes.POINTER(i)] * 3
        L.ar_oracle_tree_of_channel.argtypes = [i, i]
        L.ar_oracle_tree_allreduce.argtypes = [i, sz, i, i, i, ctypes.POINTER(vp), ctypes.POINTER(vp)]
        L.ar_oracle_tree_elements.argtypes = [i, sz, i, i, i, ctypes.POINTER(vp), vp, sz, vp]
        for name in ("ar_oracle_f32_to_bf16", "ar_oracle_f32_to_f16",
                     "ar_oracle_f16_to_f32", "ar_oracle_bf16_to_f32"):
            getattr(L, name).argtypes = [vp, vp, sz]
            getattr(L, name).restype = None
        _lib = L
    return _lib


def _check_inputs(inputs, dtype):
    st = NP_STORAGE[dtype]
    count = len(inputs[0])
    for x in inputs:
        if x.dtype != st or len(x) != count or not x.flags.c_contiguous:
            raise ValueError("oracle inputs must be contiguous %s arrays of equal length" % st)
    return count


def allreduce(inputs, dtype, op, nchannels, chunk_elems, all_ranks=False):
    """Order-matched ring AllReduce.  Returns one array (every rank's result is
    the same value) or, with all_ranks=True, the list of per-rank outputs."""
    count = _check_inputs(inputs, dtype)
    n = len(inputs)
    st = NP_STORAGE[dtype]
    vp = ctypes.c_void_p
    ins = (vp * n)(*[x.ctypes.data for x in inputs])
    if all_ranks:
        outs_np = [np.empty(count, dtype=st) for _ in range(n)]
    else:
        one = np.empty(count, dtype=st)
        outs_np = [one] * n
    outs = (vp * n)(*[o.ctypes.data for o in outs_np])
    rc = lib().ar_oracle_allreduce(n, count, DTYPES[dtype], OPS[op], nchannels, chunk_elems, ins, outs)
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return outs_np if all_ranks else outs_np[0]


def reduce_scatter(inputs, dtype, op):
    """Ring ReduceScatter: inputs[r] has N*count elements; returns the list of
    per-rank outputs (count elements each)."""
    n = len(inputs)
    total = _check_inputs(inputs, dtype)
    if total % n:
        raise ValueError("ReduceScatter inputs must hold nranks * count elements")
    count = total // n
    st = NP_STORAGE[dtype]
    outs = [np.empty(count, dtype=st) for _ in range(n)]
    vp = ctypes.c_void_p
    ins = (vp * n)(*[x.ctypes.data for x in inputs])
    outp = (vp * n)(*[o.ctypes.data for o in outs])
    if lib().ar_oracle_reduce_scatter(n, count, DTYPES[dtype], OPS[op], ins, outp) != 0:
        raise ValueError("oracle rejected the arguments")
    return outs


def all_gather(inputs, dtype):
    """AllGather: returns the list of per-rank outputs (N*count elements)."""
    n = len(inputs)
    count = _check_inputs(inputs, dtype)
    st = NP_STORAGE[dtype]
    outs = [np.empty(n * count, dtype=st) for _ in range(n)]
    vp = ctypes.c_void_p
    ins = (vp * n)(*[x.ctypes.data for x in inputs])
    outp = (vp * n)(*[o.ctypes.data for o in outs])
    if lib().ar_oracle_all_gather(n, count, ELEM_SIZE[dtype], ins, outp) != 0:
        raise ValueError("oracle rejected the arguments")
    return outs


def elements(inputs, dtype, op, nchannels, chunk_elems, idx):
    """The ring fold for the listed element indices only."""
    count = _check_inputs(inputs, dtype)
    n = len(inputs)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    res = np.empty(len(idx), dtype=NP_STORAGE[dtype])
    vp = ctypes.c_void_p
    ins = (vp * n)(*[x.ctypes.data for x in inputs])
    rc = lib().ar_oracle_elements(n, count, DTYPES[dtype], OPS[op], nchannels, chunk_elems,
                                  ins, idx.ctypes.data, len(idx), res.ctypes.data)
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return res


def locate(nranks, count, dtype, nchannels, chunk_elems, idx):
    """(channel, loop, chunk, first, length) of element idx."""
    ch, c = ctypes.c_int(), ctypes.c_int()
    lp = ctypes.c_longlong()
    first, ln = ctypes.c_size_t(), ctypes.c_size_t()
    rc = lib().ar_oracle_locate(nranks, count, DTYPES[dtype], nchannels, chunk_elems, idx,
                                ctypes.byref(ch), ctypes.byref(lp), ctypes.byref(c),
                                ctypes.byref(first), ctypes.byref(ln))
    if rc != 0:
        raise ValueError("index out of range")
    return ch.value, lp.value, c.value, first.value, ln.value


def btree(nranks, rank):
    """(up, d0, d1, child_type) of rank in the binary tree; -1 for none."""
    v = [ctypes.c_int() for _ in range(4)]
    if lib().ar_oracle_btree(nranks, rank, *[ctypes.byref(x) for x in v]) != 0:
        raise ValueError("bad rank")
    return tuple(x.value for x in v)


def dtree(nranks, rank, tree):
    """(up, d0, d1) of rank in tree 0 or 1 of the double binary tree."""
    v = [ctypes.c_int() for _ in range(3)]
    if lib().ar_oracle_dtree(nranks, rank, tree, *[ctypes.byref(x) for x in v]) != 0:
        raise ValueError("bad rank or tree")
    return tuple(x.value for x in v)


def tree_of_channel(nchannels, ch):
    t = lib().ar_oracle_tree_of_channel(nchannels, ch)
    if t < 0:
        raise ValueError("bad channel")
    return t


def tree_allreduce(inputs, dtype, op, nchannels):
    """Double-tree AllReduce; returns the one result every rank receives."""
    count = _check_inputs(inputs, dtype)
    n = len(inputs)
    one = np.empty(count, dtype=NP_STORAGE[dtype])
    vp = ctypes.c_void_p
    ins = (vp * n)(*[x.ctypes.data for x in inputs])
    outs = (vp * n)(*([one.ctypes.data] * n))
    if lib().ar_oracle_tree_allreduce(n, count, DTYPES[dtype], OPS[op], nchannels, ins, outs) != 0:
        raise ValueError("oracle rejected the arguments")
    return one


def tree_elements(inputs, dtype, op, nchannels, idx):
    """The tree fold for the listed element indices only."""
    count = _check_inputs(inputs, dtype)
    n = len(inputs)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    res = np.empty(len(idx), dtype=NP_STORAGE[dtype])
    vp = ctypes.c_void_p
    ins = (vp * n)(*[x.ctypes.data for x in inputs])
    if lib().ar_oracle_tree_elements(n, count, DTYPES[dtype], OPS[op], nchannels, ins, idx.ctypes.data,
                                     len(idx), res.ctypes.data) != 0:
        raise ValueError("oracle rejected the arguments")
    return res


def _conv(name, x, out_dtype):
    x = np.ascontiguousarray(x)
    y = np.empty(len(x), dtype=out_dtype)
    getattr(lib(), name)(x.ctypes.data, y.ctypes.data, len(x))
    return y


def f32_to_bf16(x):
    return _conv("ar_oracle_f32_to_bf16", np.asarray(x, dtype=np.float32), np.uint16)


def f32_to_f16(x):
    return _conv("ar_oracle_f32_to_f16", np.asarray(x, dtype=np.float32), np.uint16)


def f16_to_f32(x):
    return _conv("ar_oracle_f16_to_f32", np.asarray(x, dtype=np.uint16), np.float32)


def bf16_to_f32(x):
    return _conv("ar_oracle_bf16_to_f32", np.asarray(x, dtype=np.uint16), np.float32)


def to_float64(x, dtype):
    """Exact widening of stored values to float64 (int32 included)."""
    if dtype == "float16":
        return f16_to_f32(x).astype(np.float64)
    if dtype == "bfloat16":
        return bf16_to_f32(x).astype(np.float64)
    return np.asarray(x).astype(np.float64)


def direct_sum_f64(inputs, dtype, idx=None):
    """Plain float64 sum over ranks (no ring order), per element.  Exact for
    int32 inputs of the sizes used here; for floats it is the yardstick of the
    error bounds."""
    acc = None
    for x in inputs:
        v = to_float64(x if idx is None else x[idx], dtype)
        acc = v if acc is None else acc + v
    return acc


def abs_sum_f64(inputs, dtype, idx=None):
    acc = None
    for x in inputs:
        v = np.abs(to_float64(x if idx is None else x[idx], dtype))
        acc = v if acc is None else acc + v
    return acc


def gamma(n, u):
    """Higham's gamma_n = n*u / (1 - n*u): the bound on the relative error of n
    rounded additions, each with unit roundoff u."""
    return n * u / (1.0 - n * u)


UNIT_ROUNDOFF = {"float32": 2.0 ** -24, "float16": 2.0 ** -11, "bfloat16": 2.0 ** -8}


def within_tolerance(result, inputs, dtype, idx=None):
    """Bounds a correct AllReduce-Sum must meet against the float64 direct sum.

    float32: |err| <= 1e-6 * N * max|x| for every element (the stated bound).
    float16 / bfloat16: the stated "1e-2 relative" read normwise,
        ||y - s64||_2 <= 1e-2 * ||s64||_2,
    and, element by element, the bound the arithmetic itself fixes for N-1
    rounded additions: |err| <= gamma_{N-1}(u) * sum_r |x_r| with u = 2^-8
    (bfloat16) or 2^-11 (float16).  A per-element 1e-2 * sum|x| bound would
    be violated by correct bfloat16 results (gamma_7 = 0.028 at N = 8).
    int32: exact.  Returns (ok, details)."""
    n = len(inputs)
    s64 = direct_sum_f64(inputs, dtype, idx)
    y = to_float64(result, dtype)
    err = np.abs(y - s64)
    worst = float(err.max()) if len(err) else 0.0
    if dtype == "float32":
        maxabs = max(float(np.max(np.abs(to_float64(x if idx is None else x[idx], dtype))))
                     for x in inputs) if len(y) else 0.0
        bound = 1e-6 * n * maxabs
        return bool(np.all(err <= bound)), {"worst": worst, "bound": bound}
    if dtype in ("bfloat16", "float16"):
        g = gamma(max(n - 1, 0), UNIT_ROUNDOFF[dtype])
        per = g * abs_sum_f64(inputs, dtype, idx)
        ok_elem = bool(np.all(err <= per))
        norm_s = float(np.sqrt(np.sum(s64 * s64)))
        norm_e = float(np.sqrt(np.sum(err * err)))
        ok_norm = norm_e <= 1e-2 * norm_s
        return ok_elem and ok_norm, {"worst": worst, "rel_l2": norm_e / norm_s if norm_s else 0.0,
                                     "elem_ok": ok_elem}
    return bool(np.all(err == 0)), {"worst": worst}

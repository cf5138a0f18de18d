"""Pins of the CPU oracle against things other than itself: the pages' printed
worked values, closed forms, brute force on tiny inputs, an order probe whose
expected digits are derived by hand from the pages' chunk formula, and the
16-bit conversions against numpy / torch.  CPU only."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from ring_allreduce_reduction_amd import inputs as gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- worked values

@pytest.mark.parametrize("nch", [1, 2, 4])
@pytest.mark.parametrize("chunk", [4, 8, 64])
def test_worked_example_every_rank(orc, nch, chunk):
    g = _golden("worked_example.json")
    xs = [np.array(v, dtype=np.float32) for v in g["inputs"]]
    assert [list(x) for x in gen.worked_example_inputs()] == [list(x) for x in xs]
    outs = orc.allreduce(xs, "float32", "sum", nch, chunk, all_ranks=True)
    for o in outs:
        assert o.tolist() == g["expected_every_rank"]


@pytest.mark.parametrize("n", _golden("rank_marker.json")["cases_N"])
def test_rank_marker_closed_form(orc, n):
    count = 4099                       # ragged, several chunks per channel
    xs = gen.rank_marker_inputs(n, count)
    out = orc.allreduce(xs, "float32", "sum", 4, 64)
    assert out[0] == n * (n - 1) // 2
    assert not np.any(out[1:])


def test_identity_and_empty(orc):
    x = gen.make_inputs(1, 1000, "float32", seed=3)
    out = orc.allreduce(x, "float32", "sum", 3, 16)
    assert np.array_equal(out, x[0])
    xs = gen.make_inputs(5, 0, "float32")
    assert len(orc.allreduce(xs, "float32", "sum", 2, 16)) == 0


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("n", [2, 3, 5, 6])
@pytest.mark.parametrize("count", [1, 7, 16, 63, 64])
def test_int32_brute_force(orc, n, count):
    xs = gen.make_inputs(n, count, "int32", seed=n * 100 + count)
    s = np.zeros(count, dtype=np.int64)
    for x in xs:
        s += x
    for nch, chunk in [(1, 4), (2, 8), (3, 4)]:
        assert np.array_equal(orc.allreduce(xs, "int32", "sum", nch, chunk), s.astype(np.int32))
        assert np.array_equal(orc.allreduce(xs, "int32", "max", nch, chunk), np.max(xs, axis=0))
        assert np.array_equal(orc.allreduce(xs, "int32", "min", nch, chunk), np.min(xs, axis=0))


def test_int32_sum_wraps(orc):
    xs = [np.array([2 ** 31 - 1, -2 ** 31, 5, -7], dtype=np.int32),
          np.array([1, -1, 2 ** 31 - 1, -2 ** 31], dtype=np.int32),
          np.array([2 ** 30, 3, 9, 11], dtype=np.int32)]
    ref = (np.sum(np.stack(xs).astype(np.int64), axis=0) + 2 ** 31) % 2 ** 32 - 2 ** 31
    assert np.array_equal(orc.allreduce(xs, "int32", "sum", 1, 4), ref.astype(np.int32))


@pytest.mark.parametrize("n", [2, 3, 4, 6])
def test_float32_exact_rational_bound(orc, n):
    count = 61
    xs = gen.make_inputs(n, count, "float32", seed=7 + n)
    out = orc.allreduce(xs, "float32", "sum", 2, 8)
    u = Fraction(1, 2 ** 24)
    for e in range(count):
        exact = sum(Fraction(float(x[e])) for x in xs)
        mag = sum(abs(Fraction(float(x[e]))) for x in xs)
        assert abs(Fraction(float(out[e])) - exact) <= (n - 1) * u * mag


def test_float32_two_ranks_is_one_ieee_add(orc):
    xs = gen.make_inputs(2, 5000, "float32", seed=11)
    out = orc.allreduce(xs, "float32", "sum", 3, 32)
    assert np.array_equal(out, xs[0] + xs[1])          # numpy float32 add is IEEE RNE


@pytest.mark.parametrize("dtype", ["float32", "float16", "bfloat16"])
@pytest.mark.parametrize("op", ["max", "min"])
def test_float_max_min_order_free(orc, dtype, op):
    xs = gen.make_inputs(5, 999, dtype, seed=21)
    vals = np.stack([orc.to_float64(x, dtype) for x in xs])
    ref = vals.max(axis=0) if op == "max" else vals.min(axis=0)
    for nch, chunk in [(1, 8), (4, 16)]:
        got = orc.to_float64(orc.allreduce(xs, dtype, op, nch, chunk), dtype)
        assert np.array_equal(got, ref)


def test_max_keeps_incoming_on_signed_zero_tie(orc):
    # One element, one channel, two ranks: chunk 0 starts at rank 1 (acc = -0.0),
    # then rank 0's +0.0 is compared; x > acc is false, so -0.0 stays.
    xs = [np.array([0.0], dtype=np.float32), np.array([-0.0], dtype=np.float32)]
    out = orc.allreduce(xs, "float32", "max", 1, 4)
    assert np.signbit(out[0])
    out = orc.allreduce(xs, "float32", "min", 1, 4)
    assert np.signbit(out[0])


def test_fp16_two_ranks_correctly_rounded(orc):
    xs = gen.make_inputs(2, 20000, "float16", seed=5)
    a, b = (x.view(np.float16).astype(np.float64) for x in xs)
    ref = (a + b).astype(np.float16).view(np.uint16)   # exact sum, one rounding
    assert np.array_equal(orc.allreduce(xs, "float16", "sum", 1, 64), ref)


def test_bf16_two_ranks_correctly_rounded(orc):
    import torch
    xs = gen.make_inputs(2, 20000, "bfloat16", seed=6)
    a = torch.from_numpy(xs[0].view(np.int16)).view(torch.bfloat16).double()
    b = torch.from_numpy(xs[1].view(np.int16)).view(torch.bfloat16).double()
    ref = (a + b).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.allreduce(xs, "bfloat16", "sum", 2, 64), ref)


def test_fp16_ring_hops_match_numpy_half_arithmetic(orc):
    # One channel, count = N*C exactly: chunk c covers [c*C, (c+1)*C) and is
    # folded c+1, c+2, ..., c (mod N) -- numpy's float16 add rounds every hop.
    n, C = 5, 8
    xs = gen.make_inputs(n, n * C, "float16", seed=9)
    h = [x.view(np.float16) for x in xs]
    ref = np.empty(n * C, dtype=np.float16)
    for c in range(n):
        sl = slice(c * C, (c + 1) * C)
        acc = h[(c + 1) % n][sl].copy()
        for k in range(2, n + 1):
            acc = acc + h[(c + k) % n][sl]
        ref[sl] = acc
    assert np.array_equal(orc.allreduce(xs, "float16", "sum", 1, C), ref.view(np.uint16))


# ---------------------------------------------------------------- order probe

def _digits(v, n):
    d = []
    for _ in range(n):
        d.append(int(v % 16))
        v //= 16
    return d[::-1]


def _hand_chunks(count, nranks, nch, C, grain):
    """Chunk index of every element, from the pages' formulas written out with
    plain Python integers (channel share, loop, shrunk last loop)."""
    per = -(-(-(-count // nch)) // grain) * grain
    chunk_of = np.full(count, -1, dtype=np.int64)
    for ch in range(nch):
        lo, hi = min(ch * per, count), min((ch + 1) * per, count)
        off = 0
        while off < hi - lo:
            rem = hi - lo - off
            cur = C if rem >= nranks * C else -(-(-(-rem // nranks)) // grain) * grain
            for k in range(nranks):
                b, e = k * cur, min((k + 1) * cur, rem)
                if b < e:
                    chunk_of[lo + off + b: lo + off + e] = k
            off += nranks * C
    assert np.all(chunk_of >= 0)
    return chunk_of


@pytest.mark.parametrize("n,count,nch,C", [
    (2, 10, 1, 2), (3, 50, 2, 4), (4, 2, 1, 2), (5, 333, 3, 6), (8, 1000, 4, 10),
    (13, 777, 2, 8), (15, 4096, 5, 16)])
def test_order_probe_decodes_ring_order(orc, n, count, nch, C):
    xs = gen.probe_inputs(n, count)
    out = orc.allreduce(xs, "uint64", "probe", nch, C)
    chunk_of = _hand_chunks(count, n, nch, C, 2)
    for e in range(count):
        c = int(chunk_of[e])
        expect = [((c + k) % n) + 1 for k in range(1, n + 1)]   # c+1, ..., c+N-1, c
        assert _digits(int(out[e]), n) == expect, (e, c)


def test_worked_example_chunk_order(orc):
    # 4 ranks, 2 elements: with 16-byte grain (2 uint64) the shrunk chunk is 2
    # elements, so both elements are chunk 0, started by rank 1, finished by rank 0.
    out = orc.allreduce(gen.probe_inputs(4, 2), "uint64", "probe", 1, 2)
    assert _digits(int(out[0]), 4) == [2, 3, 4, 1]


# ---------------------------------------------------------------- structure

@pytest.mark.parametrize("n,count,nch,C,dtype", [
    (8, 16 * 2 ** 20 // 64, 16, 2 ** 18 // 64, "float32"),
    (72, 4099, 64, 1024, "float32"),
    (4, 777, 3, 8, "bfloat16"),
    (3, 1, 2, 4, "float32")])
def test_locate_partitions_the_buffer(orc, n, count, nch, C, dtype):
    grain = 16 // gen.ELEM_SIZE[dtype]
    chunk_of = _hand_chunks(count, n, nch, C, grain)
    seen = np.zeros(count, dtype=np.int64)
    e = 0
    while e < count:
        ch, lp, c, first, ln = orc.locate(n, count, dtype, nch, C, e)
        assert first == e and ln > 0 and c == chunk_of[e]
        seen[first:first + ln] += 1
        e = first + ln
    assert np.all(seen == 1)


def test_cfg_chunk_closed_forms(orc):
    # 72 ranks x 1Mi fp32, 64 channels: 16384 per channel, shrunk chunk 228
    _, _, _, _, ln = orc.locate(72, 2 ** 20, "float32", 64, 2 ** 18, 0)
    assert ln == 228
    # 8 ranks x 16Mi fp32, 16 channels, 1 MiB nominal chunk: one shrunk loop,
    # chunk = 1Mi/8 = 131072 elements (512 KiB)
    _, lp, c, first, ln = orc.locate(8, 16 * 2 ** 20, "float32", 16, 2 ** 18, 5 * 2 ** 20 + 3)
    assert (lp, ln) == (0, 131072) and first == 5 * 2 ** 20


def test_elements_match_full_fold(orc):
    xs = gen.make_inputs(7, 5003, "bfloat16", seed=2)
    full = orc.allreduce(xs, "bfloat16", "sum", 3, 64)
    idx = np.random.default_rng(0).integers(0, 5003, 500)
    assert np.array_equal(orc.elements(xs, "bfloat16", "sum", 3, 64, idx), full[idx])


def test_all_ranks_identical_and_inplace(orc):
    xs = gen.make_inputs(6, 3001, "float32", seed=4)
    outs = orc.allreduce(xs, "float32", "sum", 2, 32, all_ranks=True)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_float32_tolerance_vs_float64(orc):
    xs = gen.make_inputs(8, 200000, "float32", seed=0)
    out = orc.allreduce(xs, "float32", "sum", 16, 2 ** 12)
    ok, info = orc.within_tolerance(out, xs, "float32")
    assert ok, info


@pytest.mark.parametrize("dtype", ["bfloat16", "float16"])
def test_half_tolerance_vs_float64(orc, dtype):
    xs = gen.make_inputs(8, 100000, dtype, seed=1)
    out = orc.allreduce(xs, dtype, "sum", 8, 2 ** 12)
    ok, info = orc.within_tolerance(out, xs, dtype)
    assert ok, info
    assert info["rel_l2"] < 5e-3


# ---------------------------------------------------------------- conversions

def _special_f32():
    v = [0.0, -0.0, 1.0, -1.0, 65504.0, 65505.0, 65519.0, 65520.0, 1e6, -1e6,
         2.0 ** -14, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -26, 1e-30,
         float("inf"), float("-inf"), 3.4e38, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11,
         1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 2.0 ** -133, -2.0 ** -126]
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    rnd = bits.view(np.float32)
    rnd = rnd[~np.isnan(rnd)]
    return np.concatenate([np.array(v, dtype=np.float32), rnd,
                           rng.standard_normal(100000).astype(np.float32),
                           (rng.standard_normal(100000) * 1e-5).astype(np.float32)])


def test_f32_to_f16_matches_numpy(orc):
    x = _special_f32()
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(orc.f32_to_f16(x), ref)


def test_f16_to_f32_matches_numpy(orc):
    allh = np.arange(2 ** 16, dtype=np.uint32).astype(np.uint16)
    ref = allh.view(np.float16).astype(np.float32)
    got = orc.f16_to_f32(allh)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_bf16_matches_torch(orc):
    import torch
    x = _special_f32()
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.f32_to_bf16(x), ref)


def test_nan_stays_nan(orc):
    x = np.array([np.nan, -np.nan], dtype=np.float32)
    assert np.all(np.isnan(orc.f16_to_f32(orc.f32_to_f16(x))))
    assert np.all(np.isnan(orc.bf16_to_f32(orc.f32_to_bf16(x))))


# ---------------------------------------------------------------- ReduceScatter / AllGather

@pytest.mark.parametrize("n", [1, 2, 3, 6])
@pytest.mark.parametrize("count", [1, 17, 64])
def test_reduce_scatter_int_brute_force(orc, n, count):
    xs = gen.make_inputs(n, n * count, "int32", seed=n + count)
    outs = orc.reduce_scatter(xs, "int32", "sum")
    total = np.sum(np.stack(xs).astype(np.int64), axis=0).astype(np.int32)
    for r in range(n):
        assert np.array_equal(outs[r], total[r * count:(r + 1) * count])
    for op, f in (("max", np.max), ("min", np.min)):
        outs = orc.reduce_scatter(xs, "int32", op)
        ref = f(np.stack(xs), axis=0)
        for r in range(n):
            assert np.array_equal(outs[r], ref[r * count:(r + 1) * count])


@pytest.mark.parametrize("n", [2, 5, 13])
def test_reduce_scatter_order_probe(orc, n):
    # block b is folded b+1, b+2, ..., b (the reduce-scatter half of the ring)
    count = 3
    xs = gen.probe_inputs(n, n * count)
    outs = orc.reduce_scatter(xs, "uint64", "probe")
    for b in range(n):
        expect = [((b + k) % n) + 1 for k in range(1, n + 1)]
        for e in range(count):
            assert _digits(int(outs[b][e]), n) == expect


def test_reduce_scatter_fp16_hops_match_numpy(orc):
    n, count = 4, 50
    xs = gen.make_inputs(n, n * count, "float16", seed=3)
    h = [x.view(np.float16) for x in xs]
    outs = orc.reduce_scatter(xs, "float16", "sum")
    for b in range(n):
        sl = slice(b * count, (b + 1) * count)
        acc = h[(b + 1) % n][sl].copy()
        for k in range(2, n + 1):
            acc = acc + h[(b + k) % n][sl]
        assert np.array_equal(outs[b], acc.view(np.uint16))


@pytest.mark.parametrize("dtype", ["int32", "float32", "bfloat16"])
def test_all_gather_is_concatenation(orc, dtype):
    n, count = 5, 333
    xs = gen.make_inputs(n, count, dtype, seed=4)
    outs = orc.all_gather(xs, dtype)
    ref = np.concatenate(xs)
    for o in outs:
        assert np.array_equal(o, ref)


@pytest.mark.parametrize("op", ["sum", "max", "min"])
def test_allreduce_is_allgather_of_reducescatter_for_int(orc, op):
    # AllReduce = ReduceScatter + AllGather [ch.5 §四]; exact for integers
    n, count = 6, 1000
    xs = gen.make_inputs(n, n * count, "int32", seed=8)
    ag = orc.all_gather(orc.reduce_scatter(xs, "int32", op), "int32")
    ar = orc.allreduce(xs, "int32", op, 3, 64)
    for o in ag:
        assert np.array_equal(o, ar)

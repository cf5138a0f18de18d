"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle
checks.  This module holds random-number recipes only -- none of the ring
AllReduce's arithmetic -- and imports nothing else from this package.

Recipe (one independent stream per rank):
    rng_r = numpy.random.Generator(PCG64(SeedSequence([seed, r])))
    "uniform"  float32:  rng_r.uniform(-1, 1, count) rounded to float32
    "normal"   16-bit :  rng_r.standard_normal(count, dtype=float32), then
                         rounded to bfloat16 / float16 by torch's CPU cast
                         (round to nearest even) and kept as raw uint16 bits
    "int"      int32  :  rng_r.integers(-2**20, 2**20, count, endpoint=True)
"""
import numpy as np

STORAGE = {"int32": np.int32, "float32": np.float32, "float16": np.uint16,
           "bfloat16": np.uint16, "uint64": np.uint64}
ELEM_SIZE = {"int32": 4, "float32": 4, "float16": 2, "bfloat16": 2, "uint64": 8}


def rank_rng(seed: int, rank: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, rank])))


def _cast16(x32: np.ndarray, dtype: str) -> np.ndarray:
    import torch
    tdt = torch.bfloat16 if dtype == "bfloat16" else torch.float16
    return torch.from_numpy(x32).to(tdt).view(torch.int16).numpy().view(np.uint16)


def rank_input(seed: int, rank: int, count: int, dtype: str, dist: str = None) -> np.ndarray:
    """Rank `rank`'s send buffer for the given dtype (default distribution per
    dtype: float32 uniform[-1,1], 16-bit floats normal(0,1), int32 uniform
    integers in [-2^20, 2^20])."""
    rng = rank_rng(seed, rank)
    if dist is None:
        dist = {"float32": "uniform", "float16": "normal", "bfloat16": "normal",
                "int32": "int"}[dtype]
    if dtype == "int32":
        if dist != "int":
            raise ValueError("int32 inputs use the 'int' distribution")
        return rng.integers(-2 ** 20, 2 ** 20, count, endpoint=True, dtype=np.int32)
    if dist == "uniform":
        x32 = rng.uniform(-1.0, 1.0, count).astype(np.float32)
    elif dist == "normal":
        x32 = rng.standard_normal(count, dtype=np.float32)
    else:
        raise ValueError("unknown distribution %r" % dist)
    if dtype == "float32":
        return x32
    return _cast16(x32, dtype)


def make_inputs(nranks: int, count: int, dtype: str, seed: int = 0, dist: str = None):
    return [rank_input(seed, r, count, dtype, dist) for r in range(nranks)]


def worked_example_inputs():
    """The pages' demo: 4 ranks, rank r holds [r, r+1] in float32."""
    return [np.array([r, r + 1], dtype=np.float32) for r in range(4)]


def rank_marker_inputs(nranks: int, count: int):
    """Element 0 holds the rank id, every other element is 0 (float32)."""
    out = []
    for r in range(nranks):
        x = np.zeros(count, dtype=np.float32)
        if count:
            x[0] = r
        out.append(x)
    return out


def probe_inputs(nranks: int, count: int):
    """uint64 inputs x_r = r + 1 for the non-commutative order probe."""
    return [np.full(count, r + 1, dtype=np.uint64) for r in range(nranks)]

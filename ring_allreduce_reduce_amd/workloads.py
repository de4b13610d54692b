"""Seeded synthetic inputs for the ring AllReduce workloads.

This module only draws numbers; it holds none of the reduction's arithmetic.
Both the tests (for the CPU oracle and the GPU path) and the benchmark take
their inputs from here, so the two sides see identical bytes.

Recipes (value distributions of the workloads the pages and the benchmark
configurations describe):
  * ``normal``:      N(0, 1) drawn in fp32, then rounded to nearest-even into
                     the target float type (fp16/bf16/fp64 via fp32).
  * ``uniform_int``: integers uniform in [lo, hi] inclusive.
  * ``uniform``:     reals uniform in [lo, hi) drawn in fp64 (fp64) or fp32
                     (narrower types), then rounded to the target type; for
                     integer types, integers in [lo, hi] inclusive.
  * ``worked``:      the pages' worked example: rank r holds r in element 0
                     and zeros elsewhere.
Each rank's generator is numpy PCG64 seeded from a stable hash of
(key, rank), so any rank's input can be regenerated on its own.
"""
from __future__ import annotations

import hashlib

import numpy as np

# numpy storage type per dtype name; bfloat16 is carried as uint16 bits.
STORAGE = {
    "int8": np.int8,
    "int32": np.int32,
    "float16": np.float16,
    "bfloat16": np.uint16,
    "float32": np.float32,
    "float64": np.float64,
}
ELEM_BYTES = {"int8": 1, "int32": 4, "float16": 2, "bfloat16": 2, "float32": 4, "float64": 8}
FLOATS = ("float16", "bfloat16", "float32", "float64")


def seed_of(key: str, rank: int) -> int:
    h = hashlib.sha256(f"{key}|rank={rank}".encode()).digest()
    return int.from_bytes(h[:8], "little")


def _to_bf16_bits(v32: np.ndarray) -> np.ndarray:
    import torch  # torch's CPU cast rounds to nearest-even
    t = torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _cast_float(v: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bfloat16":
        return _to_bf16_bits(v.astype(np.float32))
    if dtype == "float16":
        return v.astype(np.float32).astype(np.float16)
    return v.astype(STORAGE[dtype])


def rank_input(key: str, rank: int, count: int, dtype: str, dist: str,
               lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    """Input of one rank."""
    rng = np.random.Generator(np.random.PCG64(seed_of(key, rank)))
    if dist == "worked":
        out = np.zeros(count, dtype=np.float64)
        if count:
            out[0] = rank
        if dtype in FLOATS:
            return _cast_float(out, dtype)
        return out.astype(STORAGE[dtype])
    if dist == "normal":
        return _cast_float(rng.standard_normal(count, dtype=np.float32), dtype)
    if dist == "uniform_int" or (dist == "uniform" and dtype not in FLOATS):
        return rng.integers(int(lo), int(hi), size=count, endpoint=True, dtype=STORAGE[dtype])
    if dist == "uniform":
        # fp64 draws for fp64; every narrower type draws fp32 (no 8-byte temporary)
        if dtype == "float64":
            return rng.uniform(lo, hi, size=count)
        u = rng.random(count, dtype=np.float32)
        u *= np.float32(hi - lo)
        u += np.float32(lo)
        return _cast_float(u, dtype)
    raise ValueError(f"unknown distribution {dist!r}")


def inputs(key: str, nranks: int, count: int, dtype: str, dist: str,
           lo: float = -1.0, hi: float = 1.0, threads: int = 1) -> list:
    """Every rank's input; ``threads`` > 1 draws ranks on host threads (each
    rank has its own generator, so the bytes are the same)."""
    if threads <= 1 or nranks <= 1:
        return [rank_input(key, r, count, dtype, dist, lo, hi) for r in range(nranks)]
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=min(threads, nranks)) as pool:
        return list(pool.map(lambda r: rank_input(key, r, count, dtype, dist, lo, hi), range(nranks)))


# The five workloads: (nranks, dtype, op, proto, nchannels, chunk bytes, sizes
# in bytes per rank, distribution, lo, hi).  nchannels 0 / proto None = chosen
# by the library's model.
def config1():
    return dict(nranks=4, dtype="int32", op="sum", proto="Simple", nchannels=2,
                chunk_bytes=16 * 1024, sizes=[65536 * 4], dist="uniform_int", lo=-1000, hi=1000)


def config2():
    return dict(nranks=8, dtype="float32", op="sum", proto="Simple", nchannels=16,
                chunk_bytes=512 * 1024, sizes=[64 << 20], dist="normal", lo=0, hi=0)


def config3():
    return dict(nranks=8, dtype="float32", op="sum", proto="LL", nchannels=8,
                chunk_bytes=0, sizes=[1 << s for s in range(13, 21)], dist="normal", lo=0, hi=0)


def config4():
    return dict(nranks=8, dtype="bfloat16", op="sum", proto="LL128", nchannels=0,
                chunk_bytes=0, sizes=[1 << s for s in range(20, 27)], dist="normal", lo=0, hi=0)


def config5_case(dtype: str, op: str):
    """Value range of one cell of the op x dtype grid."""
    if op == "prod" and dtype in FLOATS:
        return dict(dist="uniform", lo=0.9, hi=1.1)
    return dict(dist="uniform", lo=-4, hi=4)


CONFIG5_OPS = ("sum", "prod", "min", "max")
CONFIG5_DTYPES = ("int8", "int32", "float16", "bfloat16", "float32", "float64")
CONFIG5_SIZES = [1 << s for s in range(3, 31)]


def to_torch(arr: np.ndarray, dtype: str, device=None):
    """Tensor of `dtype` holding the stored values (bfloat16 from its bits)."""
    import torch
    if dtype == "bfloat16":
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(device) if device is not None else t


def from_torch(t, dtype: str) -> np.ndarray:
    """Stored values of a tensor as the numpy storage type of `dtype`."""
    import torch
    t = t.detach().contiguous().cpu()
    if dtype == "bfloat16":
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()

"""CPU oracle for the ring AllReduce, its two halves (ReduceScatter,
AllGather) and the double-binary-tree AllReduce: test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never imports,
links or calls it, and it imports nothing from the product.

``ring_oracle.c`` is the reduction itself (a sequential simulation of the ring
schedule, and of the tree's reduce-up / broadcast-down passes; see its
comments for the passages they follow); ``select.py`` is the
alpha-beta protocol model.  This module builds the C file with gcc and wraps it
with ctypes over numpy arrays.  bfloat16 arrays are carried as raw ``uint16``
bit patterns, since numpy has no bfloat16 type.

Parity pins (what ties this oracle to something other than itself) live in
``tests/test_oracle_pins.py`` and ``tests/test_oracle_mutations.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ring_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libring_oracle.so")

# name -> (code in ring_oracle.c, numpy storage dtype, element bytes)
DTYPES = {
    "int8": (0, np.int8, 1),
    "int32": (1, np.int32, 4),
    "float16": (2, np.float16, 2),
    "bfloat16": (3, np.uint16, 2),
    "float32": (4, np.float32, 4),
    "float64": (5, np.float64, 8),
}
OPS = {"sum": 0, "prod": 1, "min": 2, "max": 3, "avg": 4}

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle C file into a shared library (gcc, no fast-math)."""
    cmd = ["gcc", *CFLAGS, "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    sz = ctypes.c_size_t
    vp = ctypes.c_void_p
    lib.oracle_ring_allreduce.argtypes = [
        ctypes.c_int, sz, ctypes.c_int, ctypes.c_int, ctypes.c_int, sz,
        ctypes.POINTER(ctypes.c_int), ctypes.POINTER(vp), ctypes.POINTER(vp)]
    lib.oracle_ring_allreduce.restype = ctypes.c_int
    lib.oracle_ring_allreduce_channels.argtypes = [
        ctypes.c_int, sz, ctypes.c_int, ctypes.c_int, ctypes.c_int, sz,
        ctypes.POINTER(ctypes.c_int), ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_int, ctypes.c_int]
    lib.oracle_ring_allreduce_channels.restype = ctypes.c_int
    lib.oracle_element_chunks.argtypes = [sz, ctypes.c_int, ctypes.c_int, ctypes.c_int, sz, vp]
    lib.oracle_element_chunks.restype = ctypes.c_int
    lib.oracle_channel_range.argtypes = [sz, sz, ctypes.c_int, ctypes.c_int,
                                         ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.oracle_channel_range.restype = None
    lib.oracle_loop_chunk.argtypes = [sz, sz, sz, ctypes.c_int, sz]
    lib.oracle_loop_chunk.restype = sz
    lib.oracle_ring_reduce_scatter.argtypes = [
        ctypes.c_int, sz, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
        ctypes.POINTER(vp), ctypes.POINTER(vp)]
    lib.oracle_ring_reduce_scatter.restype = ctypes.c_int
    lib.oracle_ring_all_gather.argtypes = [
        ctypes.c_int, sz, sz, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(vp), ctypes.POINTER(vp)]
    lib.oracle_ring_all_gather.restype = ctypes.c_int
    ip = ctypes.POINTER(ctypes.c_int)
    lib.oracle_btree.argtypes = [ctypes.c_int, ctypes.c_int, ip, ip, ip]
    lib.oracle_btree.restype = None
    lib.oracle_dtree.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ip, ip, ip]
    lib.oracle_dtree.restype = None
    lib.oracle_tree_allreduce.argtypes = [
        ctypes.c_int, sz, ctypes.c_int, ctypes.c_int, ctypes.c_int, sz,
        ctypes.POINTER(vp), ctypes.POINTER(vp)]
    lib.oracle_tree_allreduce.restype = ctypes.c_int
    for name in ("oracle_f16_decode_array", "oracle_bf16_decode_array",
                 "oracle_f16_encode_array", "oracle_bf16_encode_array"):
        getattr(lib, name).argtypes = [vp, vp, sz]
        getattr(lib, name).restype = None
    return lib


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the oracle library, building it first if it is not there.

    With ``path`` given, load that file instead (the mutation tests load
    deliberately broken copies this way) without caching it.
    """
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = _declare(ctypes.CDLL(_LIB_PATH))
    return _lib


def _sentinel(count: int, npt) -> np.ndarray:
    """A fresh output filled with 0xA5 bytes, so an element the oracle never
    writes cannot pass for a result."""
    return np.full(count * np.dtype(npt).itemsize, 0xA5, dtype=np.uint8).view(npt)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def ring_allreduce(xs, dtype: str, op: str, nchannels: int, chunk_elems: int,
                   ring=None, lib: ctypes.CDLL | None = None, out=None):
    """Ring AllReduce of the n input arrays ``xs`` (one per rank).

    Returns the n output arrays (fresh ones unless ``out`` is given; ``out``
    may be ``xs`` itself for the in-place form).  ``ring[i]`` is the rank at
    ring index i (None = identity).  ``chunk_elems`` is the per-rank,
    per-channel chunk of a full loop and must be a multiple of 16 bytes.
    """
    lib = lib or load()
    code, npt, esize = DTYPES[dtype]
    n = len(xs)
    xs = [np.ascontiguousarray(x, dtype=npt) for x in xs]
    count = xs[0].size if n else 0
    assert all(x.size == count for x in xs)
    ys = out if out is not None else [_sentinel(count, npt) for _ in range(n)]
    xp = (ctypes.c_void_p * n)(*[_ptr(x) for x in xs])
    yp = (ctypes.c_void_p * n)(*[_ptr(y) for y in ys])
    rp = None
    if ring is not None:
        rp = (ctypes.c_int * n)(*[int(r) for r in ring])
    rc = lib.oracle_ring_allreduce(n, count, code, OPS[op], nchannels, chunk_elems, rp, xp, yp)
    if rc != 0:
        raise ValueError("oracle_ring_allreduce rejected its arguments")
    return ys


def ring_allreduce_threaded(xs, dtype: str, op: str, nchannels: int, chunk_elems: int,
                            ring=None, threads: int | None = None, lib: ctypes.CDLL | None = None,
                            out=None):
    """The same ring AllReduce as ``ring_allreduce``, with the channels spread
    over ``threads`` host threads (default: one per available core, at most
    one per channel).  Channels own disjoint element ranges, so the result is
    the same bytes; only the wall time differs.  Returns (outputs, threads
    used)."""
    from concurrent.futures import ThreadPoolExecutor

    lib = lib or load()
    code, npt, esize = DTYPES[dtype]
    n = len(xs)
    xs = [np.ascontiguousarray(x, dtype=npt) for x in xs]
    count = xs[0].size if n else 0
    assert all(x.size == count for x in xs)
    ys = out if out is not None else [_sentinel(count, npt) for _ in range(n)]
    xp = (ctypes.c_void_p * n)(*[_ptr(x) for x in xs])
    yp = (ctypes.c_void_p * n)(*[_ptr(y) for y in ys])
    rp = (ctypes.c_int * n)(*[int(r) for r in ring]) if ring is not None else None
    if threads is None:
        threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    threads = max(1, min(int(threads), nchannels))
    bounds = [(nchannels * t // threads, nchannels * (t + 1) // threads) for t in range(threads)]

    def run(b):
        return lib.oracle_ring_allreduce_channels(n, count, code, OPS[op], nchannels, chunk_elems, rp, xp, yp,
                                                  b[0], b[1])

    with ThreadPoolExecutor(max_workers=threads) as pool:
        codes = list(pool.map(run, bounds))
    if any(codes):
        raise ValueError("oracle_ring_allreduce_channels rejected its arguments")
    return ys, threads


def ring_reduce_scatter(xs, dtype: str, op: str, ring=None, lib: ctypes.CDLL | None = None, out=None):
    """Ring ReduceScatter: ``xs[r]`` holds n blocks of ``count`` elements;
    returns the n outputs of ``count`` elements (rank r: block r reduced over
    all ranks, in the ring's fold order).  ``out`` may hold views of the
    inputs' own blocks (the in-place form)."""
    lib = lib or load()
    code, npt, _ = DTYPES[dtype]
    n = len(xs)
    xs = [np.ascontiguousarray(x, dtype=npt) for x in xs]
    assert all(x.size == xs[0].size for x in xs) and xs[0].size % n == 0
    count = xs[0].size // n
    ys = out if out is not None else [_sentinel(count, npt) for _ in range(n)]
    xp = (ctypes.c_void_p * n)(*[_ptr(x) for x in xs])
    yp = (ctypes.c_void_p * n)(*[_ptr(y) for y in ys])
    rp = (ctypes.c_int * n)(*[int(r) for r in ring]) if ring is not None else None
    if lib.oracle_ring_reduce_scatter(n, count, code, OPS[op], rp, xp, yp) != 0:
        raise ValueError("oracle_ring_reduce_scatter rejected its arguments")
    return ys


def ring_all_gather(xs, dtype: str, ring=None, lib: ctypes.CDLL | None = None, out=None):
    """Ring AllGather: returns the n outputs of n blocks each (block q = rank
    q's input).  ``out`` may be the outputs whose block r is ``xs[r]``."""
    lib = lib or load()
    _, npt, esize = DTYPES[dtype]
    n = len(xs)
    xs = [np.ascontiguousarray(x, dtype=npt) for x in xs]
    count = xs[0].size
    assert all(x.size == count for x in xs)
    ys = out if out is not None else [_sentinel(n * count, npt) for _ in range(n)]
    xp = (ctypes.c_void_p * n)(*[_ptr(x) for x in xs])
    yp = (ctypes.c_void_p * n)(*[_ptr(y) for y in ys])
    rp = (ctypes.c_int * n)(*[int(r) for r in ring]) if ring is not None else None
    if lib.oracle_ring_all_gather(n, count, esize, rp, xp, yp) != 0:
        raise ValueError("oracle_ring_all_gather rejected its arguments")
    return ys


def btree(n: int, rank: int, lib: ctypes.CDLL | None = None) -> tuple[int, int, int]:
    """(parent, child slot 0, child slot 1) of ``rank`` in the binary tree
    over n ranks; -1 = none."""
    lib = lib or load()
    u, a, b = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    lib.oracle_btree(n, rank, ctypes.byref(u), ctypes.byref(a), ctypes.byref(b))
    return u.value, a.value, b.value


def dtree(n: int, rank: int, tree: int, lib: ctypes.CDLL | None = None) -> tuple[int, int, int]:
    """(parent, child slot 0, child slot 1) of ``rank`` in tree 0 or 1 of the
    double binary tree over n ranks; -1 = none."""
    lib = lib or load()
    u, a, b = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    lib.oracle_dtree(n, rank, tree, ctypes.byref(u), ctypes.byref(a), ctypes.byref(b))
    return u.value, a.value, b.value


def tree_allreduce(xs, dtype: str, op: str, nchannels: int, chunk_elems: int,
                   lib: ctypes.CDLL | None = None, out=None):
    """Tree AllReduce of the n input arrays ``xs`` over the double binary tree
    (channel c on tree c mod 2).  Returns the n outputs (fresh ones unless
    ``out`` is given; ``out`` may be ``xs`` for the in-place form)."""
    lib = lib or load()
    code, npt, _ = DTYPES[dtype]
    n = len(xs)
    xs = [np.ascontiguousarray(x, dtype=npt) for x in xs]
    count = xs[0].size if n else 0
    assert all(x.size == count for x in xs)
    ys = out if out is not None else [_sentinel(count, npt) for _ in range(n)]
    xp = (ctypes.c_void_p * n)(*[_ptr(x) for x in xs])
    yp = (ctypes.c_void_p * n)(*[_ptr(y) for y in ys])
    if lib.oracle_tree_allreduce(n, count, code, OPS[op], nchannels, chunk_elems, xp, yp) != 0:
        raise ValueError("oracle_tree_allreduce rejected its arguments")
    return ys


def element_chunks(count: int, dtype: str, nranks: int, nchannels: int,
                   chunk_elems: int, lib: ctypes.CDLL | None = None) -> np.ndarray:
    """Chunk id (0..n-1) of every element under the oracle's partition."""
    lib = lib or load()
    out = np.empty(count, dtype=np.int32)
    rc = lib.oracle_element_chunks(count, DTYPES[dtype][0], nranks, nchannels, chunk_elems,
                                   _ptr(out) if count else None)
    if rc != 0:
        raise ValueError("oracle_element_chunks rejected its arguments")
    return out


def channel_range(count: int, dtype: str, nchannels: int, c: int) -> tuple[int, int]:
    lib = load()
    lo, hi = ctypes.c_size_t(), ctypes.c_size_t()
    lib.oracle_channel_range(count, DTYPES[dtype][2], nchannels, c, ctypes.byref(lo), ctypes.byref(hi))
    return lo.value, hi.value


def loop_chunk(length: int, off: int, dtype: str, nranks: int, chunk_elems: int) -> int:
    return load().oracle_loop_chunk(length, off, DTYPES[dtype][2], nranks, chunk_elems)


def f16_decode(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.size, dtype=np.float32)
    load().oracle_f16_decode_array(_ptr(bits), _ptr(out), bits.size)
    return out


def f16_encode(vals: np.ndarray) -> np.ndarray:
    vals = np.ascontiguousarray(vals, dtype=np.float32)
    out = np.empty(vals.size, dtype=np.uint16)
    load().oracle_f16_encode_array(_ptr(vals), _ptr(out), vals.size)
    return out


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.size, dtype=np.float32)
    load().oracle_bf16_decode_array(_ptr(bits), _ptr(out), bits.size)
    return out


def bf16_encode(vals: np.ndarray) -> np.ndarray:
    vals = np.ascontiguousarray(vals, dtype=np.float32)
    out = np.empty(vals.size, dtype=np.uint16)
    load().oracle_bf16_encode_array(_ptr(vals), _ptr(out), vals.size)
    return out

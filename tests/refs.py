"""Independent references that pin the CPU oracle.

Nothing here calls the oracle's arithmetic: every value is computed with numpy
or torch CPU routines (library arithmetic in the element type), with the
element -> chunk map as the only input taken from the oracle's partition
(which itself is pinned by literal tables in tests/golden/).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import torch

from ring_allreduce_reduce_amd.workloads import FLOATS, STORAGE

EPS = {"float16": 2.0 ** -10, "bfloat16": 2.0 ** -7, "float32": 2.0 ** -23, "float64": 2.0 ** -52}


def bf16_bits_to_torch(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def torch_to_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values to float64."""
    if dtype == "bfloat16":
        return bf16_bits_to_torch(a).to(torch.float64).numpy()
    return np.asarray(a).astype(np.float64)


def hop(dtype: str, op: str, a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """op(received a, local b) elementwise, computed by numpy/torch in the
    element type (16-bit floats: torch/numpy compute in fp32, round back)."""
    if dtype == "bfloat16":
        ta, tb = bf16_bits_to_torch(a), bf16_bits_to_torch(b)
        if op == "sum":
            r = ta + tb
        elif op == "prod":
            r = ta * tb
        elif op == "min":
            r = torch.where(tb < ta, tb, ta)
        else:
            r = torch.where(tb > ta, tb, ta)
        return torch_to_bf16_bits(r)
    a = np.asarray(a, dtype=STORAGE[dtype])
    b = np.asarray(b, dtype=STORAGE[dtype])
    with np.errstate(over="ignore"):
        if op == "sum":
            return (a + b).astype(STORAGE[dtype])
        if op == "prod":
            return (a * b).astype(STORAGE[dtype])
    if op == "min":
        return np.where(b < a, b, a)
    return np.where(b > a, b, a)


def divide(dtype: str, a: np.ndarray, n: int) -> np.ndarray:
    """a / n elementwise in the element type: integers truncate toward zero
    (exact integer arithmetic), floats divide in numpy / torch (16-bit floats
    compute in fp32 and round to nearest-even)."""
    if dtype == "bfloat16":
        return torch_to_bf16_bits(bf16_bits_to_torch(a) / n)
    if dtype in ("int8", "int32"):
        w = np.asarray(a).astype(np.int64)
        q = np.abs(w) // n * np.sign(w)
        return q.astype(STORAGE[dtype])
    a = np.asarray(a, dtype=STORAGE[dtype])
    return (a / np.asarray(n, dtype=STORAGE[dtype])).astype(STORAGE[dtype])


def hop_op(op: str) -> str:
    """The per-hop operation: avg folds like sum."""
    return "sum" if op == "avg" else op


def exact_reduce(xs, dtype: str, op: str) -> np.ndarray:
    """The plain definition for the order-free cases (integers with
    wraparound, min and max of anything): numpy's reduction over ranks."""
    X = np.stack(xs)
    if dtype == "bfloat16":
        assert op in ("min", "max")
        t = bf16_bits_to_torch(X.reshape(-1)).reshape(X.shape)
        r = t.min(dim=0).values if op == "min" else t.max(dim=0).values
        return torch_to_bf16_bits(r)
    with np.errstate(over="ignore"):
        if op == "sum":
            return np.sum(X, axis=0, dtype=STORAGE[dtype])
        if op == "prod":
            return np.prod(X, axis=0, dtype=STORAGE[dtype])
    return X.min(axis=0) if op == "min" else X.max(axis=0)


def fold_closed_form(xs, dtype: str, op: str, chunk_of: np.ndarray, ring=None) -> np.ndarray:
    """Per-element result of passing chunk k once around the ring: it starts
    at ring index k+1 and every later ring index folds its own value in as the
    local operand, so acc = x[k+1]; acc = op(acc, x[k+j]) for j = 2..n."""
    n = len(xs)
    ring = list(range(n)) if ring is None else list(ring)
    X = np.stack(xs)
    cols = np.arange(X.shape[1])
    order = np.asarray(ring)
    acc = X[order[(chunk_of + 1) % n], cols]
    for j in range(2, n + 1):
        acc = hop(dtype, op, acc, X[order[(chunk_of + j) % n], cols])
    return acc


def error_bound_ok(y: np.ndarray, xs, dtype: str, op: str, idx: np.ndarray) -> bool:
    """|y - exact| <= (n-1) eps sum|x| (sum), or (n-1) eps prod|x| (prod), at the
    sampled elements; the exact value uses fsum / rational arithmetic."""
    n = len(xs)
    X = np.stack([to_f64(x, dtype) for x in xs])
    yv = to_f64(y, dtype)
    eps = EPS[dtype]
    for e in idx:
        col = [float(v) for v in X[:, e]]
        if op == "sum":
            exact = math.fsum(col)
            bound = (n - 1) * eps * math.fsum(abs(v) for v in col)
            if abs(yv[e] - exact) > bound:
                return False
        else:
            exact = Fraction(1)
            for v in col:
                exact *= Fraction(v)
            mag = abs(exact)
            bound = Fraction((n - 1) * eps) * mag * Fraction(1 + n * eps)
            if abs(Fraction(float(yv[e])) - exact) > bound:
                return False
    return True


def all_equal(ys) -> bool:
    return all(np.array_equal(ys[0].view(np.uint8), y.view(np.uint8)) for y in ys[1:])

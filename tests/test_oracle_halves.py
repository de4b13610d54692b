"""Pins of the oracle's ReduceScatter and AllGather against things other than
themselves (CPU only).

* Order-free ReduceScatter (integers, min, max): numpy's reduction of block r
  over ranks.
* Float ReduceScatter with n = 2: one IEEE operation computed by numpy/torch.
* Float fold order: a threaded brute-force ring with real FIFOs whose messages
  carry the rank of their block, cut into channel and loop pieces (which must
  not change any result), on tiny inputs.
* ReduceScatter is the first half of the ring AllReduce: with the identity
  ring and one chunk per block, rank r's ReduceScatter output equals block r
  of the (separately pinned) AllReduce oracle's output.
* The error bound of the pages' reduction for floats.
* AllGather: numpy concatenation, bit for bit; the brute-force ring.
* Invariants: in place equals out of place, n = 1 copies.
"""
import numpy as np
import pytest

import oracle
from bruteforce_ring import run_all_gather as brute_ag
from bruteforce_ring import run_reduce_scatter as brute_rs
from refs import error_bound_ok, exact_reduce, hop
from ring_allreduce_reduce_amd import workloads as W

DTYPES = list(W.STORAGE)
OPS = ["sum", "prod", "min", "max"]


def _gen(key, n, count, dtype, op):
    if dtype in W.FLOATS and op == "prod":
        return W.inputs(key, n, count, dtype, "uniform", 0.9, 1.1)
    return W.inputs(key, n, count, dtype, "uniform", -4, 4)


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("n,count", [(1, 7), (2, 5), (3, 33), (5, 1), (8, 100)])
def test_reduce_scatter_order_free_equals_numpy(dtype, op, n, count):
    if dtype in W.FLOATS and op in ("sum", "prod"):
        pytest.skip("order-dependent; pinned by the brute-force ring and the n = 2 case")
    xs = _gen(f"rs-free-{dtype}-{op}-{n}", n, n * count, dtype, op)
    ring = list(np.random.default_rng(n).permutation(n))
    ys = oracle.ring_reduce_scatter(xs, dtype, op, ring=ring)
    full = exact_reduce(xs, dtype, op)
    for r in range(n):
        assert np.array_equal(_bits(ys[r]), _bits(full[r * count:(r + 1) * count])), r


@pytest.mark.parametrize("dtype", list(W.FLOATS))
@pytest.mark.parametrize("op", ["sum", "prod"])
def test_reduce_scatter_two_ranks_is_one_operation(dtype, op):
    xs = _gen(f"rs-two-{dtype}-{op}", 2, 2 * 301, dtype, op)
    for ring in ([0, 1], [1, 0]):
        ys = oracle.ring_reduce_scatter(xs, dtype, op, ring=ring)
        full = hop(dtype, op, xs[0], xs[1])     # one operation, commutative
        for r in range(2):
            assert np.array_equal(_bits(ys[r]), _bits(full[r * 301:(r + 1) * 301]))


def _cases(seed, k):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(k):
        n = int(rng.integers(1, 6))
        count = int(rng.integers(0, 40))
        nch = int(rng.integers(1, 4))
        units = int(rng.integers(1, 4))
        dtype = DTYPES[int(rng.integers(0, len(DTYPES)))]
        op = OPS[int(rng.integers(0, 4))]
        ring = [int(v) for v in rng.permutation(n)]
        out.append((n, count, nch, units, dtype, op, ring))
    return out


@pytest.mark.parametrize("case", _cases(77, 80), ids=lambda c: "-".join(map(str, c[:6])))
def test_reduce_scatter_bruteforce_ring(case):
    n, count, nch, units, dtype, op, ring = case
    xs = _gen(f"rs-brute-{case}", n, n * count, dtype, op)
    want = brute_rs(xs, dtype, op, nch, units * 16 // W.ELEM_BYTES[dtype], ring)
    got = oracle.ring_reduce_scatter(xs, dtype, op, ring=ring)
    for g, w in zip(got, want):
        assert np.array_equal(_bits(g), _bits(w))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("op", OPS)
def test_reduce_scatter_is_the_first_half_of_allreduce(dtype, op):
    n = 6
    count = 3 * 16 // W.ELEM_BYTES[dtype]          # one block = one 16-byte aligned chunk
    xs = _gen(f"rs-half-{dtype}-{op}", n, n * count, dtype, op)
    ar = oracle.ring_allreduce(xs, dtype, op, 1, count)
    rs = oracle.ring_reduce_scatter(xs, dtype, op)
    for r in range(n):
        assert np.array_equal(_bits(rs[r]), _bits(ar[0][r * count:(r + 1) * count])), r


@pytest.mark.parametrize("dtype", list(W.FLOATS))
@pytest.mark.parametrize("op", ["sum", "prod"])
def test_reduce_scatter_error_bound(dtype, op):
    n, count = 8, 400
    xs = W.inputs(f"rs-bound-{dtype}-{op}", n, n * count, dtype, "normal") if op == "sum" else \
        W.inputs(f"rs-bound-{dtype}-{op}", n, n * count, dtype, "uniform", 0.9, 1.1)
    ys = oracle.ring_reduce_scatter(xs, dtype, op)
    for r in (0, 5):
        idx = np.random.default_rng(r).choice(count, size=60, replace=False)
        blocks = [x[r * count:(r + 1) * count] for x in xs]
        assert error_bound_ok(ys[r], blocks, dtype, op, idx)


@pytest.mark.parametrize("dtype", DTYPES)
def test_reduce_scatter_in_place(dtype):
    n, count = 4, 29
    xs = _gen(f"rs-inplace-{dtype}", n, n * count, dtype, "sum")
    ring = [2, 0, 3, 1]
    want = oracle.ring_reduce_scatter(xs, dtype, "sum", ring=ring)
    bufs = [x.copy() for x in xs]
    outs = [bufs[r][r * count:(r + 1) * count] for r in range(n)]
    oracle.ring_reduce_scatter(bufs, dtype, "sum", ring=ring, out=outs)
    for w, o in zip(want, outs):
        assert np.array_equal(_bits(w), _bits(o))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n,count", [(1, 9), (2, 0), (3, 17), (8, 1000)])
def test_all_gather_equals_concatenation(dtype, n, count):
    xs = W.inputs(f"ag-{dtype}-{n}", n, count, dtype, "uniform", -4, 4)
    ring = list(np.random.default_rng(n + 1).permutation(n))
    ys = oracle.ring_all_gather(xs, dtype, ring=ring)
    cat = np.concatenate(xs) if n else np.zeros(0)
    for y in ys:
        assert np.array_equal(_bits(y), _bits(cat))


@pytest.mark.parametrize("case", _cases(91, 40), ids=lambda c: "-".join(map(str, c[:5])))
def test_all_gather_bruteforce_ring(case):
    n, count, nch, units, dtype, _, ring = case
    xs = W.inputs(f"ag-brute-{case}", n, count, dtype, "uniform", -4, 4)
    want = brute_ag(xs, dtype, nch, units * 16 // W.ELEM_BYTES[dtype], ring)
    got = oracle.ring_all_gather(xs, dtype, ring=ring)
    for g, w in zip(got, want):
        assert np.array_equal(_bits(g), _bits(w))


def test_all_gather_in_place():
    n, count = 5, 13
    xs = W.inputs("ag-inplace", n, count, "int32", "uniform", -4, 4)
    ys = [np.zeros(n * count, dtype=np.int32) for _ in range(n)]
    for r in range(n):
        ys[r][r * count:(r + 1) * count] = xs[r]
    ins = [ys[r][r * count:(r + 1) * count] for r in range(n)]
    oracle.ring_all_gather(ins, "int32", ring=[4, 2, 0, 1, 3], out=ys)
    for y in ys:
        assert np.array_equal(y, np.concatenate(xs))


def test_halves_reject_bad_arguments():
    lib = oracle.load()
    assert lib.oracle_ring_reduce_scatter(0, 4, 4, 0, None, None, None) == -1
    assert lib.oracle_ring_reduce_scatter(2, 4, 9, 0, None, None, None) == -1
    assert lib.oracle_ring_all_gather(2, 4, 0, None, None, None) == -1

"""Parity of the HIP ring ReduceScatter and AllGather (through the C ABI) with
the CPU oracle, bit for bit.

ReduceScatter: every dtype and op under the three protocols, n = 2, 3, 8,
blocks with and without a ragged 16-byte tail (a block length that is not a
multiple of 16 bytes also misaligns every block start, which takes the
element-wise path), several channel counts and chunk sizes (several loops),
ring orders, in place, the straight-line and the general kernel form, and a
large call.  AllGather: the same shapes; its result is a plain concatenation.
"""
import numpy as np
import pytest
import torch

import oracle
import ring_allreduce_reduce_amd as ra
from ring_allreduce_reduce_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
DTYPES = list(W.STORAGE)
PROTOS = ["LL", "LL128", "Simple"]


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


def _gen(key, n, count, dtype, op):
    if dtype in W.FLOATS and op == "prod":
        return W.inputs(key, n, count, dtype, "uniform", 0.9, 1.1)
    return W.inputs(key, n, count, dtype, "uniform", -4, 4)


def _sync_code():
    torch.cuda.synchronize()
    return ra.ringar_get_async_error(torch.cuda.current_stream().cuda_stream)


def run_rs(xs, dtype, op, proto="auto", nch=0, chunk_bytes=0, ring=None, inplace=False, **cfg):
    n = len(xs)
    count = xs[0].size // n
    print(f"reduce_scatter n={n} block={count} {dtype} {op} {proto} nch={nch} chunk={chunk_bytes} "
          f"ring={ring} inplace={inplace} {cfg}", flush=True)
    sends = [W.to_torch(x, dtype, DEV) for x in xs]
    recvs = [s[r * count:(r + 1) * count] for r, s in enumerate(sends)] if inplace else \
        [torch.full((count,), 0, dtype=sends[0].dtype, device=DEV) for _ in range(n)]
    ra.reduce_scatter(sends, recvs, op=op, nchannels=nch, proto=proto, chunk_bytes=chunk_bytes,
                      ring_order=ring, **cfg)
    code = _sync_code()
    assert code == ra.SUCCESS, ra.ringar_result_string(code)
    got = [W.from_torch(r, dtype) for r in recvs]
    want = oracle.ring_reduce_scatter(xs, dtype, op, ring=ring)
    for r, (g, w) in enumerate(zip(got, want)):
        if not np.array_equal(_bits(g), _bits(w)):
            bad = np.nonzero(_bits(g) != _bits(w))[0][:8] // W.ELEM_BYTES[dtype]
            pytest.fail(f"rank {r}: differs from the oracle at elements {bad}")
    if not inplace:
        for x, s in zip(xs, sends):
            assert np.array_equal(_bits(x), _bits(W.from_torch(s, dtype))), "send buffer modified"


def run_ag(xs, dtype, proto="auto", nch=0, chunk_bytes=0, ring=None, inplace=False, **cfg):
    n = len(xs)
    count = xs[0].size
    print(f"all_gather n={n} count={count} {dtype} {proto} nch={nch} chunk={chunk_bytes} ring={ring} "
          f"inplace={inplace} {cfg}", flush=True)
    if inplace:
        recvs = [torch.full((n * count,), 0, dtype=W.to_torch(xs[0], dtype, DEV).dtype, device=DEV)
                 for _ in range(n)]
        for r in range(n):
            recvs[r][r * count:(r + 1) * count] = W.to_torch(xs[r], dtype, DEV)
        sends = [recvs[r][r * count:(r + 1) * count] for r in range(n)]
    else:
        sends = [W.to_torch(x, dtype, DEV) for x in xs]
        recvs = [torch.full((n * count,), 0, dtype=sends[0].dtype, device=DEV) for _ in range(n)]
    ra.all_gather(sends, recvs, nchannels=nch, proto=proto, chunk_bytes=chunk_bytes, ring_order=ring, **cfg)
    code = _sync_code()
    assert code == ra.SUCCESS, ra.ringar_result_string(code)
    cat = np.concatenate([np.ascontiguousarray(x) for x in xs])
    want = oracle.ring_all_gather(xs, dtype, ring=ring)
    for r, rv in enumerate(recvs):
        g = W.from_torch(rv, dtype)
        assert np.array_equal(_bits(want[r]), _bits(cat))
        if not np.array_equal(_bits(g), _bits(cat)):
            bad = np.nonzero(_bits(g) != _bits(cat))[0][:8] // W.ELEM_BYTES[dtype]
            pytest.fail(f"rank {r}: differs at elements {bad}")


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("dtype", DTYPES)
def test_reduce_scatter_every_op(proto, dtype):
    for j, op in enumerate(["sum", "prod", "min", "max"]):
        for n, block in [(2, 4099), (3, 16 * 64 + 16 // W.ELEM_BYTES[dtype]), (8, 2000 + j)]:
            xs = _gen(f"rs-{proto}-{dtype}-{op}-{n}", n, n * block, dtype, op)
            ring = list(np.random.default_rng(n + j).permutation(n)) if j % 2 else None
            run_rs(xs, dtype, op, proto, nch=1 + j, ring=ring)


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("form", ["auto", "general"])
def test_reduce_scatter_loops_and_lanes(proto, form):
    # small chunks: several loops per channel; ragged last loop; several lanes
    for (n, block, nch, units, lanes) in [(5, 12345, 3, 64, 0), (8, 50000, 2, 256, 4), (4, 777, 1, 1, 0),
                                          (6, 1 << 16, 4, 1024, 0)]:
        xs = _gen(f"rs-loops-{proto}-{n}-{block}", n, n * block, "float32", "sum")
        run_rs(xs, "float32", "sum", proto, nch, units * 16, ring=list(range(n))[::-1], lanes=lanes,
               force_general=int(form == "general"))


@pytest.mark.parametrize("proto", PROTOS)
def test_reduce_scatter_in_place(proto):
    for dtype in ("bfloat16", "int32", "float64"):
        xs = _gen(f"rs-ip-{proto}-{dtype}", 6, 6 * 3001, dtype, "sum")
        run_rs(xs, dtype, "sum", proto, 3, ring=[3, 1, 5, 0, 2, 4], inplace=True)


def test_reduce_scatter_large():
    # 8 ranks, 64 MiB of input per rank (8 MiB blocks), the 16-channel Simple shape
    n, block = 8, 2 << 20
    xs = _gen("rs-large", n, n * block, "float32", "sum")
    run_rs(xs, "float32", "sum", "Simple", 16, 512 * 1024)


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("dtype", DTYPES)
def test_all_gather(proto, dtype):
    for j, (n, count, nch) in enumerate([(2, 1, 1), (3, 4099, 2), (8, 2048, 4), (5, 33333, 3)]):
        xs = W.inputs(f"ag-{proto}-{dtype}-{n}", n, count, dtype, "uniform", -4, 4)
        ring = list(np.random.default_rng(j).permutation(n)) if j % 2 else None
        run_ag(xs, dtype, proto, nch, ring=ring)


@pytest.mark.parametrize("proto", PROTOS)
@pytest.mark.parametrize("form", ["auto", "general"])
def test_all_gather_in_place_and_loops(proto, form):
    for (n, count, nch, units) in [(4, 10000, 2, 64), (7, 999, 1, 1), (8, 1 << 15, 4, 256)]:
        xs = W.inputs(f"ag-ip-{proto}-{n}", n, count, "float16", "uniform", -4, 4)
        run_ag(xs, "float16", proto, nch, units * 16, ring=list(range(n))[::-1], inplace=True,
               force_general=int(form == "general"))


def test_all_gather_large():
    n, count = 8, 2 << 20          # 8 MiB per rank, 64 MiB output per rank
    xs = W.inputs("ag-large", n, count, "float32", "normal")
    run_ag(xs, "float32", "Simple", 16, 512 * 1024)


def test_halves_one_rank_and_empty():
    xs = _gen("rs-one", 1, 100, "float32", "sum")
    run_rs(xs, "float32", "sum", "Simple", 2)
    run_ag(W.inputs("ag-one", 1, 100, "int8", "uniform", -4, 4), "int8", "LL", 1)
    s = [torch.zeros(8, device=DEV) for _ in range(3)]
    r = [torch.zeros(0, device=DEV) for _ in range(3)]
    ra.reduce_scatter([torch.zeros(0, device=DEV)] * 3, r)
    assert _sync_code() == ra.SUCCESS
    del s


def test_halves_timeout_when_a_rank_never_runs():
    n, block = 4, 4096
    sends = [torch.ones(n * block, device=DEV) for _ in range(n)]
    recvs = [torch.zeros(block, device=DEV) for _ in range(n)]
    ra.reduce_scatter(sends, recvs, nchannels=2, proto="LL", skip_rank=2, spin_limit_ms=20)
    assert _sync_code() == ra.TIMEOUT
    # the library recovers: the next call is correct
    ra.reduce_scatter(sends, recvs, nchannels=2, proto="LL")
    assert _sync_code() == ra.SUCCESS
    assert all(bool((r == n).all()) for r in recvs)

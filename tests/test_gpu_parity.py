"""Parity of the HIP ring AllReduce (through the C ABI) with the CPU oracle.

Bit-exact everywhere: the GPU path must reproduce the oracle's ring fold
order for floats and the exact result for integers, min and max.  Covers the
five workloads (int32 Simple, 64 MiB fp32 Simple at 16 channels, the LL
sweep, the bf16 LL128 sweep with automatic channels, the op x dtype grid with
automatic protocol), ragged and empty inputs, in-place calls, ring orders,
unaligned buffers, repeated calls that reuse FIFO memory, and the timeout and
abort paths (forced from the host, every kernel exits normally).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import ring_allreduce_reduce_amd as ra
from libutil import oracle_model
from oracle import select as S
from refs import error_bound_ok, exact_reduce
from ring_allreduce_reduce_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
DTYPES = list(W.STORAGE)


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


def run_gpu(xs, dtype, op, proto="auto", nch=0, chunk_bytes=0, ring=None, inplace=False, lanes=0,
            **cfg):
    n = len(xs)
    count = xs[0].size
    sends = [W.to_torch(x, dtype, DEV) for x in xs]
    recvs = sends if inplace else [torch.full_like(s, 0) for s in sends]
    ra.allreduce(sends, recvs, op=op, nchannels=nch, proto=proto, chunk_bytes=chunk_bytes,
                 ring_order=ring, lanes=lanes, **cfg)
    torch.cuda.synchronize()
    code = ra.ringar_get_async_error(torch.cuda.current_stream().cuda_stream)
    plan = ra.ringar_plan(count, dtype, n, nch, proto, ra.make_config(chunk_bytes=chunk_bytes, lanes=lanes))
    outs = [W.from_torch(r, dtype) for r in recvs]
    ins_after = [W.from_torch(s, dtype) for s in sends] if not inplace else None
    return outs, plan, code, ins_after


def check(xs, dtype, op, proto="auto", nch=0, chunk_bytes=0, ring=None, inplace=False, lanes=0, **cfg):
    print(f"case n={len(xs)} count={xs[0].size} {dtype} {op} {proto} nch={nch} chunk={chunk_bytes} "
          f"ring={ring} inplace={inplace} lanes={lanes} {cfg}", flush=True)
    outs, plan, code, after = run_gpu(xs, dtype, op, proto, nch, chunk_bytes, ring, inplace, lanes, **cfg)
    assert code == ra.SUCCESS, ra.ringar_result_string(code)
    want = oracle.ring_allreduce(xs, dtype, op, plan.nchannels, plan.chunk_elems, ring=ring)
    for r, (g, w) in enumerate(zip(outs, want)):
        if not np.array_equal(_bits(g), _bits(w)):
            bad = np.nonzero(_bits(g).reshape(-1, W.ELEM_BYTES[dtype]).any(axis=1) !=
                             _bits(w).reshape(-1, W.ELEM_BYTES[dtype]).any(axis=1))[0][:5]
            diff = np.nonzero((_bits(g) != _bits(w)))[0][:8] // W.ELEM_BYTES[dtype]
            pytest.fail(f"rank {r}: differs from the oracle at elements {diff} (zero pattern {bad})")
    if after is not None:
        for x, a in zip(xs, after):
            assert np.array_equal(_bits(x), _bits(a)), "send buffer modified"
    return outs, plan


# ------------------------------------------------------------ the workloads
def test_config1_int32_simple():
    c = W.config1()
    count = c["sizes"][0] // 4
    xs = W.inputs("config1", c["nranks"], count, c["dtype"], c["dist"], c["lo"], c["hi"])
    outs, plan = check(xs, c["dtype"], c["op"], c["proto"], c["nchannels"], c["chunk_bytes"])
    assert (plan.proto, plan.nchannels, plan.chunk_elems) == (2, 2, 4096)
    ref = exact_reduce(xs, "int32", "sum")
    for o in outs:
        assert np.array_equal(o, ref)


def test_config2_fp32_64MiB_simple_16ch():
    c = W.config2()
    count = c["sizes"][0] // 4
    xs = W.inputs("config2", c["nranks"], count, c["dtype"], c["dist"])
    outs, plan = check(xs, c["dtype"], c["op"], c["proto"], c["nchannels"], c["chunk_bytes"])
    assert (plan.proto, plan.nchannels, plan.chunk_bytes) == (2, 16, 512 * 1024)
    idx = np.random.default_rng(1).choice(count, size=2000, replace=False)
    assert error_bound_ok(outs[0], xs, "float32", "sum", idx)


@pytest.mark.parametrize("nbytes", W.config3()["sizes"])
def test_config3_ll_sweep(nbytes):
    c = W.config3()
    xs = W.inputs(f"config3-{nbytes}", c["nranks"], nbytes // 4, c["dtype"], c["dist"])
    _, plan = check(xs, c["dtype"], c["op"], c["proto"], c["nchannels"])
    assert (plan.proto, plan.nchannels) == (0, 8)


@pytest.mark.parametrize("nbytes", W.config4()["sizes"])
def test_config4_ll128_bf16_sweep(nbytes):
    c = W.config4()
    xs = W.inputs(f"config4-{nbytes}", c["nranks"], nbytes // 2, c["dtype"], c["dist"])
    _, plan = check(xs, c["dtype"], c["op"], c["proto"], c["nchannels"])
    assert plan.proto == 1
    assert plan.nchannels == S.auto_channels(oracle_model(), 8, "LL128", nbytes)


@pytest.mark.parametrize("dtype", W.CONFIG5_DTYPES)
@pytest.mark.parametrize("op", W.CONFIG5_OPS)
def test_config5_grid_up_to_1MiB(dtype, op):
    om = oracle_model()
    es = W.ELEM_BYTES[dtype]
    for nbytes in [s for s in W.CONFIG5_SIZES if s <= (1 << 20) and s >= es]:
        count = nbytes // es
        rng = W.config5_case(dtype, op)
        xs = W.inputs(f"config5-{dtype}-{op}-{nbytes}", 8, count, dtype, rng["dist"], rng["lo"], rng["hi"])
        _, plan = check(xs, dtype, op)
        want = S.resolve(om, 8, nbytes)
        assert (ra.PROTO_NAMES[plan.proto], plan.nchannels, plan.chunk_bytes) == want


BIG_SIZES = [1 << s for s in range(21, 30)]          # 2 MiB .. 512 MiB per rank
GRID = [(op, dt) for op in W.CONFIG5_OPS for dt in W.CONFIG5_DTYPES]
# every grid cell at one size between 2 and 512 MiB (each size covered at
# least twice over the grid), every cell at 64 MiB, and at the grid's
# largest size (1 GiB per rank) every cell of the 1-, 4- and 8-byte types and
# one of the 16-bit floats (the oracle's 16-bit codec takes minutes there)
LARGE = [(op, dt, BIG_SIZES[j % 9]) for j, (op, dt) in enumerate(GRID) if BIG_SIZES[j % 9] != 64 << 20] + \
    [(op, dt, 64 << 20) for op, dt in GRID] + \
    [(op, dt, 1 << 30) for op in W.CONFIG5_OPS for dt in ("int8", "int32", "float32", "float64")] + \
    [("prod", "bfloat16", 1 << 30)]
HOST_THREADS = 16


@pytest.mark.parametrize("case", LARGE, ids=[f"{o}-{d}-{b >> 20}MiB" for o, d, b in LARGE])
def test_config5_grid_large_sizes(case):
    """The op x dtype grid above 1 MiB per rank, up to 1 GiB, automatic
    protocol and channels, compared element by element with the oracle
    (inputs drawn and the oracle run on host threads; ranks copied back and
    compared one at a time)."""
    op, dtype, nbytes = case
    om = oracle_model()
    es = W.ELEM_BYTES[dtype]
    count = nbytes // es
    rng = W.config5_case(dtype, op)
    print(f"case grid {op} {dtype} {nbytes} bytes per rank", flush=True)
    xs = W.inputs(f"config5-{dtype}-{op}-{nbytes}", 8, count, dtype, rng["dist"], rng["lo"], rng["hi"],
                  threads=HOST_THREADS)
    sends = [W.to_torch(x, dtype, DEV) for x in xs]
    recvs = [torch.empty_like(t) for t in sends]
    ra.allreduce(sends, recvs, op=op)
    torch.cuda.synchronize()
    assert ra.ringar_get_async_error(torch.cuda.current_stream().cuda_stream) == 0
    plan = ra.ringar_plan(count, dtype, 8)
    assert (ra.PROTO_NAMES[plan.proto], plan.nchannels, plan.chunk_bytes) == S.resolve(om, 8, nbytes)
    del sends
    torch.cuda.empty_cache()
    want, _ = oracle.ring_allreduce_threaded(xs, dtype, op, plan.nchannels, plan.chunk_elems,
                                             threads=HOST_THREADS)
    del xs
    for r in range(8):
        got = W.from_torch(recvs[r], dtype)
        assert np.array_equal(_bits(got), _bits(want[r])), (op, dtype, nbytes, r)
        del got
    del recvs, want
    torch.cuda.empty_cache()


# ------------------------------------------------------------ edge cases
RAGGED = [  # (n, count, nch, chunk units of 16 B, lanes)
    (2, 1, 1, 1, 0), (3, 17, 2, 1, 0), (5, 1000, 3, 2, 0), (8, 4099, 4, 3, 0), (7, 65537, 2, 64, 0),
    (4, 300001, 3, 0, 0), (8, 1 << 18, 16, 0, 8), (6, 123457, 5, 1000, 4), (8, 999, 64, 1, 0),
    (2, 2 ** 20 + 3, 1, 0, 32), (3, 50000, 1, 7, 2),
]


@pytest.mark.parametrize("form", ["auto", "general"])
@pytest.mark.parametrize("proto", ["LL", "LL128", "Simple"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_ragged_shapes(proto, dtype, form):
    # "auto" runs the straight-line form wherever the lane parts allow it,
    # "general" forces the general form on the same shapes
    for i, (n, count, nch, units, lanes) in enumerate(RAGGED):
        xs = W.inputs(f"ragged-{proto}-{dtype}-{i}", n, count, dtype, "uniform", -4, 4)
        ring = list(np.random.default_rng(i).permutation(n)) if i % 2 else None
        check(xs, dtype, "sum" if i % 3 else "max", proto, nch, units * 16, ring=ring, lanes=lanes,
              force_general=int(form == "general"))


@pytest.mark.parametrize("proto", ["LL", "Simple"])
@pytest.mark.parametrize("n", [2, 3, 8])
def test_small_form_every_op_and_dtype(proto, n):
    # one 16-byte packet per lane and step: counts with and without a ragged
    # last packet, in place and out of place
    for dtype in DTYPES:
        es = W.ELEM_BYTES[dtype]
        for j, op in enumerate(W.CONFIG5_OPS):
            count = (n * 64 * 16 // es) * (j + 1) // 3 + (j % 2) * 3 + 1
            dist = ("uniform", 0.9, 1.1) if op == "prod" and es > 1 and dtype != "int32" else ("uniform", -4, 4)
            xs = W.inputs(f"small-{proto}-{dtype}-{op}-{n}", n, count, dtype, *dist)
            outs, plan = check(xs, dtype, op, proto, 1, 0, inplace=bool(j % 2))
            assert plan.small_slices == 1, (dtype, op, count, plan.lanes)


# a chunk of four slots per lane at depth 8, two at depth 4, one at depth 2
SLOT_BYTES = {"LL": 8192, "LL128": 30720, "Simple": 32768}


@pytest.mark.parametrize("depth", [2, 4, 8])
@pytest.mark.parametrize("proto", ["LL", "LL128", "Simple"])
def test_every_fifo_depth(proto, depth):
    chunk = 4 * SLOT_BYTES[proto]
    lanes = 8 // depth
    n, nch = 5, 3
    count = nch * n * (chunk // 4) * 2 + 777     # two loops per channel and a ragged tail
    xs = W.inputs("depth", n, count, "float32", "normal")
    outs, plan = check(xs, "float32", "sum", proto, nch, chunk, lanes=lanes, fifo_depth=depth)
    assert (plan.lanes, plan.nchannels) == (lanes, nch)


@pytest.mark.parametrize("proto", ["LL", "LL128", "Simple"])
def test_inplace_equals_out_of_place(proto):
    xs = W.inputs(f"inplace-{proto}", 8, 200003, "float32", "normal")
    a, _ = check(xs, "float32", "sum", proto, 5, 0)
    b, _ = check(xs, "float32", "sum", proto, 5, 0, inplace=True)
    for x, y in zip(a, b):
        assert np.array_equal(_bits(x), _bits(y))


def test_unaligned_buffers_take_the_elementwise_path():
    n, count = 4, 10007
    for dtype in ["int8", "float16", "float32", "float64"]:
        es = W.ELEM_BYTES[dtype]
        xs = W.inputs(f"unal-{dtype}", n, count, dtype, "uniform", -4, 4)
        for proto in ["LL", "LL128", "Simple"]:
            big = [W.to_torch(np.concatenate([np.zeros(1, x.dtype), x]), dtype, DEV) for x in xs]
            sends = [b[1:] for b in big]                     # one element past an aligned start
            recvs = [torch.zeros(count + 1, dtype=b.dtype, device=DEV)[1:] for b in big]
            assert sends[0].data_ptr() % 16 == es % 16
            ra.allreduce(sends, recvs, op="sum", nchannels=3, proto=proto)
            torch.cuda.synchronize()
            assert ra.ringar_get_async_error(torch.cuda.current_stream().cuda_stream) == 0
            plan = ra.ringar_plan(count, dtype, n, 3, proto)
            want = oracle.ring_allreduce(xs, dtype, "sum", plan.nchannels, plan.chunk_elems)
            for r in range(n):
                assert np.array_equal(_bits(W.from_torch(recvs[r], dtype)), _bits(want[r])), (dtype, proto, r)


def test_repeated_calls_reuse_fifo_memory():
    # many calls, shapes and protocols on one stream: stale flags or counters
    # from an earlier call must never be taken for fresh data
    rng = np.random.default_rng(11)
    for it in range(24):
        proto = ["LL", "LL128", "Simple"][it % 3]
        n = int(rng.integers(2, 9))
        count = int(rng.integers(1, 300000))
        nch = int(rng.integers(1, 9))
        dtype = DTYPES[int(rng.integers(0, 6))]
        xs = W.inputs(f"repeat-{it}", n, count, dtype, "uniform", -4, 4)
        check(xs, dtype, "sum", proto, nch, 0)


def test_one_rank_and_empty():
    xs = W.inputs("one", 1, 1000, "float32", "normal")
    outs, _ = check(xs, "float32", "sum", "Simple", 1)
    assert np.array_equal(outs[0], xs[0])
    s = [torch.ones(0, device=DEV) for _ in range(4)]
    ra.allreduce(s, [torch.ones(0, device=DEV) for _ in range(4)])
    torch.cuda.synchronize()


def test_worked_example_on_gpu():
    for n in (2, 4, 8):
        xs = W.inputs("worked", n, 32 * 1024 * 1024 if n == 8 else 4096, "float32", "worked")
        outs, _, code, _ = run_gpu(xs, "float32", "sum", "Simple", 16, 512 * 1024)
        assert code == 0
        for o in outs:
            assert o[0] == n * (n - 1) // 2 and not np.any(o[1:])


# ------------------------------------------------------------ failure paths
def test_timeout_when_a_rank_never_runs():
    xs = W.inputs("skip", 4, 100000, "float32", "normal")
    for proto in ["LL", "LL128", "Simple"]:
        outs, _, code, _ = run_gpu(xs, "float32", "sum", proto, 2, skip_rank=2, spin_limit_ms=20)
        assert code == ra.TIMEOUT, (proto, ra.ringar_result_string(code))
    # the next call on the same stream is unaffected
    check(xs, "float32", "sum", "Simple", 2)
    check(xs, "float32", "sum", "LL", 2)


def test_abort_flag_ends_waits():
    flag = torch.ones(1, dtype=torch.int32).pin_memory()
    xs = W.inputs("abort", 4, 50000, "float32", "normal")
    outs, _, code, _ = run_gpu(xs, "float32", "sum", "Simple", 2, skip_rank=1, spin_limit_ms=60000,
                               abort_flag=flag.data_ptr())
    assert code == ra.ABORTED
    check(xs, "float32", "sum", "Simple", 2)


@pytest.mark.parametrize("n", [9, 16, 33, 64])
def test_many_ranks(n):
    """Up to the library's 64 ranks: 2(n-1) stages per loop, every protocol,
    ragged counts, and a ring order that is not the identity."""
    for j, proto in enumerate(["LL", "LL128", "Simple"]):
        xs = W.inputs(f"many-{n}-{proto}", n, 20011 + 7 * j, "float32", "normal")
        ring = list(np.random.default_rng(n).permutation(n)) if j == 1 else None
        check(xs, "float32", "sum", proto, 2, 0, ring=ring)

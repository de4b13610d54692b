"""Parity of the direct form of the ring AllReduce (Simple, each slice
written straight into the successor's receive buffer) with the CPU oracle.

The direct form changes where the data travels, not the fold order, so the
results must equal the ring oracle's bit for bit: ragged shapes over several
loops, lanes and channel counts, every op and dtype, unaligned buffers, the
in-place fallback to FIFOs, calls that alternate with the FIFO form on one
stream, the 64 MiB workload, the timeout and abort paths, and the library's
own choice of the direct form for calls whose protocol the model picks.
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


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


def run(xs, dtype, op, nch, chunk_bytes=0, lanes=0, inplace=False, direct=1, **cfg):
    n, count = len(xs), xs[0].size
    print(f"case direct={direct} n={n} count={count} {dtype} {op} nch={nch} chunk={chunk_bytes} lanes={lanes} "
          f"inplace={inplace} {cfg}", flush=True)
    sends = [W.to_torch(x, dtype, DEV) for x in xs]
    recvs = sends if inplace else [torch.full_like(s, 0) for s in sends]
    ra.allreduce(sends, recvs, op=op, nchannels=nch, proto="Simple", chunk_bytes=chunk_bytes, lanes=lanes,
                 direct=direct, **cfg)
    torch.cuda.synchronize()
    code = ra.ringar_get_async_error(torch.cuda.current_stream().cuda_stream)
    plan = ra.ringar_plan(count, dtype, n, nch, "Simple",
                          ra.make_config(chunk_bytes=chunk_bytes, lanes=lanes, direct=direct))
    return [W.from_torch(r, dtype) for r in recvs], plan, code, [W.from_torch(s, dtype) for s in sends]


def check(xs, dtype, op, nch, chunk_bytes=0, lanes=0, inplace=False, direct=1, **cfg):
    outs, plan, code, after = run(xs, dtype, op, nch, chunk_bytes, lanes, inplace, direct, **cfg)
    assert code == ra.SUCCESS, ra.ringar_result_string(code)
    assert plan.direct == direct
    want = oracle.ring_allreduce(xs, dtype, op, plan.nchannels, plan.chunk_elems)
    for r, (g, w) in enumerate(zip(outs, want)):
        if not np.array_equal(_bits(g), _bits(w)):
            diff = np.nonzero(_bits(g) != _bits(w))[0][:8] // W.ELEM_BYTES[dtype]
            pytest.fail(f"rank {r}: differs from the oracle at elements {diff}")
    if not inplace:
        for x, a in zip(xs, after):
            assert np.array_equal(_bits(x), _bits(a)), "send buffer modified"
    return outs, plan


def test_workload_64MiB():
    xs = W.inputs("config2", 8, 16 << 20, "float32", "normal")
    check(xs, "float32", "sum", 16, 512 * 1024)


RAGGED = [  # (n, count, nch, chunk units of 16 B, lanes)
    (2, 1, 1, 1, 0), (3, 17, 2, 1, 0), (5, 1000, 3, 2, 0), (8, 4099, 4, 3, 0), (7, 65537, 2, 64, 0),
    (4, 300001, 3, 0, 0), (8, 1 << 18, 16, 0, 8), (6, 123457, 5, 1000, 4), (8, 999, 64, 1, 0),
    (2, 2 ** 20 + 3, 1, 0, 32), (3, 50000, 1, 7, 2), (16, 77777, 2, 0, 0), (8, 3 << 20, 2, 4096, 0),
]


@pytest.mark.parametrize("dtype", DTYPES)
def test_ragged_shapes(dtype):
    for i, (n, count, nch, units, lanes) in enumerate(RAGGED):
        xs = W.inputs(f"direct-ragged-{dtype}-{i}", n, count, dtype, "uniform", -4, 4)
        check(xs, dtype, "sum" if i % 3 else "max", nch, units * 16, lanes)


@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32", "float64"])
def test_every_op(dtype):
    for op in W.CONFIG5_OPS:
        dist = ("uniform", 0.9, 1.1) if op == "prod" and dtype not in ("int32",) else ("uniform", -4, 4)
        xs = W.inputs(f"direct-ops-{dtype}-{op}", 8, 400009, dtype, *dist)
        check(xs, dtype, op, 6, 16384)


def test_unaligned_buffers():
    n, count = 4, 10007
    for dtype in ["int8", "float16", "float32", "float64"]:
        xs = W.inputs(f"direct-unal-{dtype}", n, count, dtype, "uniform", -4, 4)
        big = [W.to_torch(np.concatenate([np.zeros(1, x.dtype), x]), dtype, DEV) for x in xs]
        sends = [b[1:] for b in big]
        recvs = [torch.zeros(count + 1, dtype=b.dtype, device=DEV)[1:] for b in big]
        ra.allreduce(sends, recvs, op="sum", nchannels=3, proto="Simple", direct=1)
        torch.cuda.synchronize()
        assert ra.ringar_get_async_error(torch.cuda.current_stream().cuda_stream) == 0
        plan = ra.ringar_plan(count, dtype, n, 3, "Simple", ra.make_config(direct=1))
        want = oracle.ring_allreduce(xs, dtype, "sum", plan.nchannels, plan.chunk_elems)
        for r in range(n):
            assert np.array_equal(_bits(W.from_torch(recvs[r], dtype)), _bits(want[r])), (dtype, r)


def test_in_place_falls_back_to_fifos():
    xs = W.inputs("direct-inplace", 8, 200003, "float32", "normal")
    a, _ = check(xs, "float32", "sum", 5)
    b, _ = check(xs, "float32", "sum", 5, inplace=True)
    for x, y in zip(a, b):
        assert np.array_equal(_bits(x), _bits(y))


def test_calls_alternate_with_the_fifo_form():
    rng = np.random.default_rng(9)
    for it in range(20):
        n = int(rng.integers(2, 9))
        count = int(rng.integers(1, 400000))
        nch = int(rng.integers(1, 9))
        dtype = DTYPES[int(rng.integers(0, 6))]
        xs = W.inputs(f"direct-mix-{it}", n, count, dtype, "uniform", -4, 4)
        check(xs, dtype, "sum", nch, direct=it % 2)


def test_timeout_when_a_rank_never_runs():
    xs = W.inputs("direct-skip", 4, 100000, "float32", "normal")
    _, _, code, _ = run(xs, "float32", "sum", 2, skip_rank=2, spin_limit_ms=20)
    assert code == ra.TIMEOUT, ra.ringar_result_string(code)
    check(xs, "float32", "sum", 2)


def test_abort_flag_ends_waits():
    flag = torch.ones(1, dtype=torch.int32).pin_memory()
    xs = W.inputs("direct-abort", 4, 50000, "float32", "normal")
    _, _, code, _ = run(xs, "float32", "sum", 2, skip_rank=1, spin_limit_ms=60000, abort_flag=flag.data_ptr())
    assert code == ra.ABORTED
    check(xs, "float32", "sum", 2)


@pytest.mark.parametrize("nbytes", [256 << 10, 4 << 20, 64 << 20])
def test_library_choice_of_the_direct_form(nbytes):
    # proto AUTO with direct = 0: the library takes the direct form where the
    # model takes Simple on the ring; in place keeps the FIFOs; both match
    # the oracle bit for bit, and so does the same call forced to FIFOs
    n, count = 8, nbytes // 4
    xs = W.inputs(f"direct-auto-{nbytes}", n, count, "float32", "normal")
    plan = ra.ringar_plan(count, "float32", n, 0, "auto")
    assert plan.direct == int(ra.PROTO_NAMES[plan.proto] == "Simple"), (nbytes, plan.proto)
    want = oracle.ring_allreduce(xs, "float32", "sum", plan.nchannels, plan.chunk_elems)
    for inplace, direct in ((False, 0), (True, 0), (False, 2)):
        print(f"case library direct choice {nbytes} inplace={inplace} direct={direct} plan.direct={plan.direct}",
              flush=True)
        sends = [W.to_torch(x, "float32", DEV) for x in xs]
        recvs = sends if inplace else [torch.zeros_like(s) for s in sends]
        ra.allreduce(sends, recvs, op="sum", nchannels=0, proto="auto", direct=direct)
        torch.cuda.synchronize()
        assert ra.ringar_get_async_error(torch.cuda.current_stream().cuda_stream) == ra.SUCCESS
        for r in range(n):
            assert np.array_equal(_bits(W.from_torch(recvs[r], "float32")), _bits(want[r])), (inplace, direct, r)

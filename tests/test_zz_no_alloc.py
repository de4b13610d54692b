"""The allocation-free AllReduce (ringar_allreduce_noalloc: FIFO slots,
counters and error word in the library's fixed scratch array) against the
allocating one (ringar_allreduce_ex) through the C ABI: bit for bit on the
same inputs and arguments, and against the oracle, on calls in a row whose
later ones are smaller, across protocols (the scratch is cleared when the
protocol changes), the tree, the direct form and in place; a call whose
connections cannot fit is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import oracle
import ring_allreduce_reduce_amd as ra
from ring_allreduce_reduce_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


def _run(fn, xs, dtype, op, n, nch, proto, cfg, st, inplace=False):
    sends = [W.to_torch(x, dtype, DEV) for x in xs]
    recvs = sends if inplace else [torch.full_like(s, 0) for s in sends]
    count = xs[0].size
    with torch.cuda.stream(st):
        code = fn([t.data_ptr() for t in sends], [t.data_ptr() for t in recvs], count, dtype, op, n, nch, proto,
                  st.cuda_stream, cfg)
    st.synchronize()
    assert code == ra.SUCCESS, (fn.__name__, ra.ringar_result_string(code), ra.ringar_last_error())
    assert ra.ringar_get_async_error(st.cuda_stream) == ra.SUCCESS
    return [W.from_torch(t, dtype) for t in recvs]


# (n, count, dtype, op, proto, nchannels, algorithm, direct, in place); each
# later call smaller than the first, protocols changing from call to call
CALLS = [
    (8, 1 << 20, "float32", "sum", "Simple", 8, "ring", 0, False),    # lanes cut to fit the scratch
    (8, 300007, "bfloat16", "sum", "LL128", 4, "ring", 0, False),
    (8, 65537, "float32", "avg", "LL", 8, "ring", 0, True),
    (5, 200003, "int8", "max", "Simple", 3, "ring", 1, False),        # direct form
    (8, 100003, "float16", "prod", "LL128", 4, "tree", 0, False),
    (4, 4099, "float64", "min", "LL", 2, "ring", 0, False),
    (8, 1000, "float32", "sum", "Simple", 1, "ring", 0, False),       # small-slice form
]


def _case(i, call, st):
    n, count, dtype, op, proto, nch, algo, direct, inplace = call
    print(f"case no-alloc {i}: {call}", flush=True)
    lo, hi = (0.9, 1.1) if (op == "prod" and dtype in W.FLOATS) else (-4, 4)
    xs = W.inputs(f"noalloc-{i}", n, count, dtype, "uniform", lo, hi)
    cfg = ra.make_config(algo=algo, direct=direct)
    got = _run(ra.ringar_allreduce_noalloc, xs, dtype, op, n, nch, proto, cfg, st, inplace)
    ref = _run(ra.ringar_allreduce_ex, xs, dtype, op, n, nch, proto, cfg, st, inplace)
    for r in range(n):
        assert np.array_equal(_bits(got[r]), _bits(ref[r])), (i, r)
    plan = ra.ringar_plan(count, dtype, n, nch, proto, cfg)
    run = oracle.tree_allreduce if plan.algo == 1 else oracle.ring_allreduce
    want = run(xs, dtype, op, plan.nchannels, plan.chunk_elems)
    for r in range(n):
        assert np.array_equal(_bits(got[r]), _bits(want[r])), (i, r)


def test_noalloc_equals_allocating_entry_point_two_calls_second_smaller():
    st = torch.cuda.Stream()
    _case(0, CALLS[0], st)
    _case(1, CALLS[1], st)


def test_noalloc_sequence_of_protocols_and_forms():
    st = torch.cuda.Stream()
    for i, call in enumerate(CALLS):
        _case(10 + i, call, st)
    # back on the first shape after the others: what they left must not leak
    _case(20, CALLS[0], st)


def test_noalloc_refuses_what_the_scratch_cannot_hold():
    st = torch.cuda.Stream()
    n, count = 8, 1 << 24                     # 64 MiB per rank, 32 channels of 512 KiB chunks
    xs = [torch.zeros(count, device=DEV) for _ in range(n)]
    ys = [torch.zeros(count, device=DEV) for _ in range(n)]
    code = ra.ringar_allreduce_noalloc([t.data_ptr() for t in xs], [t.data_ptr() for t in ys], count, "float32",
                                       "sum", n, 32, "Simple", st.cuda_stream, ra.make_config(chunk_bytes=512 << 10))
    assert code == ra.INVALID_USAGE
    assert "scratch" in ra.ringar_last_error()
    # a forced lane count that does not fit is refused too
    code = ra.ringar_allreduce_noalloc([t.data_ptr() for t in xs], [t.data_ptr() for t in ys], 1 << 20, "float32",
                                       "sum", n, 8, "Simple", st.cuda_stream, ra.make_config(lanes=32))
    assert code == ra.INVALID_USAGE
    st.synchronize()
    assert ra.ringar_get_async_error(st.cuda_stream) == ra.SUCCESS

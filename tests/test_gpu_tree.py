"""Parity of the HIP tree AllReduce (through the C ABI) with the CPU oracle.

Bit-exact everywhere: the GPU path must reproduce the oracle's tree fold order
(own input, then child 0, then child 1, channel c on tree c % 2) for floats
and the exact result for integers, min and max.  Covers the three protocols
and both kernel forms on ragged shapes, every op and dtype, every FIFO depth,
deep trees (up to 64 ranks), in-place calls, calls that share FIFO memory
with the ring, the model's automatic choice of algorithm, the 64 MiB
workload, and the timeout and abort paths (forced from the host, every
kernel exits normally).
"""
import numpy as np
import pytest
import torch

import oracle
import ring_allreduce_reduce_amd as ra
from refs import error_bound_ok, exact_reduce
from ring_allreduce_reduce_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
DTYPES = list(W.STORAGE)


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


def run_tree(xs, dtype, op, proto="auto", nch=0, chunk_bytes=0, inplace=False, lanes=0, algo="tree", **cfg):
    n = len(xs)
    count = xs[0].size
    sends = [W.to_torch(x, dtype, DEV) for x in xs]
    recvs = sends if inplace else [torch.full_like(s, 0) for s in sends]
    ra.allreduce(sends, recvs, op=op, nchannels=nch, proto=proto, chunk_bytes=chunk_bytes, lanes=lanes,
                 algo=algo, **cfg)
    torch.cuda.synchronize()
    code = ra.ringar_get_async_error(torch.cuda.current_stream().cuda_stream)
    plan = ra.ringar_plan(count, dtype, n, nch, proto,
                          ra.make_config(chunk_bytes=chunk_bytes, lanes=lanes, algo=algo,
                                         fifo_depth=cfg.get("fifo_depth", 0)))
    outs = [W.from_torch(r, dtype) for r in recvs]
    after = [W.from_torch(s, dtype) for s in sends] if not inplace else None
    return outs, plan, code, after


def check(xs, dtype, op, proto="auto", nch=0, chunk_bytes=0, inplace=False, lanes=0, algo="tree", **cfg):
    print(f"case tree n={len(xs)} count={xs[0].size} {dtype} {op} {proto} nch={nch} chunk={chunk_bytes} "
          f"inplace={inplace} lanes={lanes} algo={algo} {cfg}", flush=True)
    outs, plan, code, after = run_tree(xs, dtype, op, proto, nch, chunk_bytes, inplace, lanes, algo, **cfg)
    assert code == ra.SUCCESS, ra.ringar_result_string(code)
    if plan.algo == 1:
        want = oracle.tree_allreduce(xs, dtype, op, plan.nchannels, plan.chunk_elems)
    else:
        want = oracle.ring_allreduce(xs, dtype, op, plan.nchannels, plan.chunk_elems)
    for r, (g, w) in enumerate(zip(outs, want)):
        if not np.array_equal(_bits(g), _bits(w)):
            diff = np.nonzero(_bits(g) != _bits(w))[0][:8] // W.ELEM_BYTES[dtype]
            pytest.fail(f"rank {r}: differs from the oracle at elements {diff}")
    if after is not None:
        for x, a in zip(xs, after):
            assert np.array_equal(_bits(x), _bits(a)), "send buffer modified"
    return outs, plan


def test_workload_64MiB_fp32_simple_16ch():
    c = W.config2()
    count = c["sizes"][0] // 4
    xs = W.inputs("config2", c["nranks"], count, c["dtype"], c["dist"])
    outs, plan = check(xs, c["dtype"], c["op"], c["proto"], c["nchannels"], c["chunk_bytes"])
    assert (plan.algo, plan.proto, plan.nchannels) == (1, 2, 16)
    idx = np.random.default_rng(1).choice(count, size=2000, replace=False)
    assert error_bound_ok(outs[0], xs, "float32", "sum", idx)


RAGGED = [  # (n, count, nch, chunk units of 16 B, lanes)
    (2, 1, 1, 1, 0), (3, 17, 2, 1, 0), (5, 1000, 3, 2, 0), (8, 4099, 4, 3, 0), (7, 65537, 2, 64, 0),
    (4, 300001, 3, 0, 0), (8, 1 << 18, 16, 0, 8), (6, 123457, 5, 1000, 4), (8, 999, 64, 1, 0),
    (2, 2 ** 20 + 3, 1, 0, 32), (3, 50000, 1, 7, 2), (16, 77777, 2, 0, 0),
]


@pytest.mark.parametrize("form", ["auto", "general"])
@pytest.mark.parametrize("proto", ["LL", "LL128", "Simple"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_ragged_shapes(proto, dtype, form):
    for i, (n, count, nch, units, lanes) in enumerate(RAGGED):
        xs = W.inputs(f"tree-ragged-{proto}-{dtype}-{i}", n, count, dtype, "uniform", -4, 4)
        check(xs, dtype, "sum" if i % 3 else "max", proto, nch, units * 16, lanes=lanes,
              force_general=int(form == "general"), inplace=bool(i % 4 == 1))


# The split form (Simple, 256 KiB per channel or more): ragged tails, chunks
# that leave odd slice sizes (the halves cut at 16-byte units), forced lanes
# and FIFO depths.  (n, channels, KiB per channel, tail elements, chunk units
# of 16 B, lanes, FIFO depth)
SPLIT = [
    (2, 1, 300, 3, 0, 0, 0), (3, 2, 256, 1, 100, 1, 0), (5, 3, 400, 5, 0, 0, 4), (8, 2, 512, 9, 777, 2, 0),
    (8, 4, 260, 15, 0, 0, 8), (16, 1, 300, 1, 0, 0, 2), (6, 1, 1024, 7, 301, 4, 2), (8, 1, 256, 0, 0, 0, 0),
]


@pytest.mark.parametrize("dtype", DTYPES)
def test_split_form_ragged(dtype):
    es = W.ELEM_BYTES[dtype]
    for i, (n, nch, kib, tail, units, lanes, depth) in enumerate(SPLIT):
        count = (kib << 10) * nch // es + tail
        op = W.CONFIG5_OPS[i % len(W.CONFIG5_OPS)]
        dist = ("uniform", 0.9, 1.1) if op == "prod" and dtype in W.FLOATS else ("uniform", -4, 4)
        xs = W.inputs(f"tree-split-{dtype}-{i}", n, count, dtype, *dist)
        outs, plan = check(xs, dtype, op, "Simple", nch, units * 16, lanes=lanes, fifo_depth=depth,
                           inplace=bool(i % 3 == 2))
        assert plan.tree_split == 1, (n, nch, kib, units, lanes)


@pytest.mark.parametrize("proto", ["LL", "Simple"])
@pytest.mark.parametrize("n", [2, 3, 8])
def test_small_form_every_op_and_dtype(proto, n):
    for dtype in DTYPES:
        es = W.ELEM_BYTES[dtype]
        for j, op in enumerate(W.CONFIG5_OPS):
            count = (64 * 16 // es) * (j + 1) // 2 + (j % 2) * 3 + 1
            dist = ("uniform", 0.9, 1.1) if op == "prod" and es > 1 and dtype != "int32" else ("uniform", -4, 4)
            xs = W.inputs(f"tree-small-{proto}-{dtype}-{op}-{n}", n, count, dtype, *dist)
            outs, plan = check(xs, dtype, op, proto, 2, 0, inplace=bool(j % 2))
            assert plan.small_slices == 1, (dtype, op, count, plan.lanes)


@pytest.mark.parametrize("proto", ["LL", "LL128", "Simple"])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
def test_every_op_general_form(proto, dtype):
    for op in W.CONFIG5_OPS:
        dist = ("uniform", 0.9, 1.1) if op == "prod" and dtype != "int32" else ("uniform", -4, 4)
        xs = W.inputs(f"tree-ops-{proto}-{dtype}-{op}", 8, 300007, dtype, *dist)
        check(xs, dtype, op, proto, 6, 0)


SLOT_BYTES = {"LL": 8192, "LL128": 30720, "Simple": 32768}


@pytest.mark.parametrize("depth", [2, 4, 8])
@pytest.mark.parametrize("proto", ["LL", "LL128", "Simple"])
def test_every_fifo_depth(proto, depth):
    chunk = 4 * SLOT_BYTES[proto]
    lanes = 8 // depth
    n, nch = 5, 3
    count = nch * (chunk // 4) * 3 + 777     # three chunks per channel and a ragged tail
    xs = W.inputs("tree-depth", n, count, "float32", "normal")
    outs, plan = check(xs, "float32", "sum", proto, nch, chunk, lanes=lanes, fifo_depth=depth)
    assert (plan.lanes, plan.nchannels, plan.fifo_depth) == (lanes, nch, depth)


@pytest.mark.parametrize("n", [9, 16, 31, 33, 64])
def test_deep_trees(n):
    for proto in ["LL", "LL128", "Simple"]:
        xs = W.inputs(f"tree-deep-{n}-{proto}", n, 20011, "float32", "normal")
        check(xs, "float32", "sum", proto, 2, 0)


@pytest.mark.parametrize("proto", ["LL", "LL128", "Simple"])
def test_inplace_equals_out_of_place(proto):
    xs = W.inputs(f"tree-inplace-{proto}", 8, 200003, "float32", "normal")
    a, _ = check(xs, "float32", "sum", proto, 5, 0)
    b, _ = check(xs, "float32", "sum", proto, 5, 0, inplace=True)
    for x, y in zip(a, b):
        assert np.array_equal(_bits(x), _bits(y))


def test_calls_alternate_with_the_ring():
    # tree and ring calls on one stream share the FIFO memory and counters:
    # stale flags or counters of the other algorithm must never pass for
    # fresh data
    rng = np.random.default_rng(5)
    for it in range(24):
        proto = ["LL", "LL128", "Simple"][it % 3]
        algo = ["tree", "ring"][(it // 3) % 2]
        n = int(rng.integers(2, 9))
        count = int(rng.integers(1, 300000))
        nch = int(rng.integers(1, 9))
        dtype = DTYPES[int(rng.integers(0, 6))]
        xs = W.inputs(f"tree-mix-{it}", n, count, dtype, "uniform", -4, 4)
        check(xs, dtype, "sum", proto, nch, 0, algo=algo)


def test_auto_algorithm_runs_what_the_plan_says():
    for nbytes in [8, 1 << 12, 1 << 16, 1 << 20, 1 << 24]:
        xs = W.inputs(f"tree-auto-{nbytes}", 8, nbytes // 4, "float32", "normal")
        check(xs, "float32", "sum", "auto", 0, 0, algo="auto")


def test_integer_sum_is_exact():
    xs = W.inputs("tree-int", 8, 1 << 20, "int32", "uniform_int", -1000, 1000)
    outs, _ = check(xs, "int32", "sum", "Simple", 4, 16384)
    ref = exact_reduce(xs, "int32", "sum")
    assert all(np.array_equal(o, ref) for o in outs)


def test_one_rank_and_empty():
    xs = W.inputs("tree-one", 1, 1000, "float32", "normal")
    outs, _ = check(xs, "float32", "sum", "Simple", 1)
    assert np.array_equal(outs[0], xs[0])
    s = [torch.ones(0, device=DEV) for _ in range(4)]
    ra.allreduce(s, [torch.ones(0, device=DEV) for _ in range(4)], algo="tree")
    torch.cuda.synchronize()


def test_worked_example_on_gpu():
    for n in (2, 4, 8):
        xs = W.inputs("worked", n, 32 * 1024 * 1024 if n == 8 else 4096, "float32", "worked")
        outs, _, code, _ = run_tree(xs, "float32", "sum", "Simple", 16, 512 * 1024)
        assert code == 0
        for o in outs:
            assert o[0] == n * (n - 1) // 2 and not np.any(o[1:])


def test_large_256MiB_per_rank():
    count = (256 << 20) // 4
    xs = W.inputs("tree-256MiB", 8, count, "float32", "normal")
    outs, plan = check(xs, "float32", "sum", "Simple", 16, 0)
    assert plan.algo == 1


def test_timeout_when_a_rank_never_runs():
    xs = W.inputs("tree-skip", 4, 100000, "float32", "normal")
    for proto in ["LL", "LL128", "Simple"]:
        _, _, code, _ = run_tree(xs, "float32", "sum", proto, 2, skip_rank=2, spin_limit_ms=20)
        assert code == ra.TIMEOUT, (proto, ra.ringar_result_string(code))
    check(xs, "float32", "sum", "Simple", 2)
    check(xs, "float32", "sum", "LL", 2)


def test_abort_flag_ends_waits():
    flag = torch.ones(1, dtype=torch.int32).pin_memory()
    xs = W.inputs("tree-abort", 4, 50000, "float32", "normal")
    _, _, code, _ = run_tree(xs, "float32", "sum", "Simple", 2, skip_rank=1, spin_limit_ms=60000,
                             abort_flag=flag.data_ptr())
    assert code == ra.ABORTED
    check(xs, "float32", "sum", "Simple", 2)


def test_unaligned_buffers_take_the_elementwise_path():
    n, count = 5, 10007
    for dtype in ["int8", "float16", "float32", "float64"]:
        xs = W.inputs(f"tree-unal-{dtype}", n, count, dtype, "uniform", -4, 4)
        for proto in ["LL", "LL128", "Simple"]:
            big = [W.to_torch(np.concatenate([np.zeros(1, x.dtype), x]), dtype, DEV) for x in xs]
            sends = [b[1:] for b in big]
            recvs = [torch.zeros(count + 1, dtype=b.dtype, device=DEV)[1:] for b in big]
            ra.allreduce(sends, recvs, op="sum", nchannels=3, proto=proto, algo="tree")
            torch.cuda.synchronize()
            assert ra.ringar_get_async_error(torch.cuda.current_stream().cuda_stream) == 0
            plan = ra.ringar_plan(count, dtype, n, 3, proto, ra.make_config(algo="tree"))
            want = oracle.tree_allreduce(xs, dtype, "sum", plan.nchannels, plan.chunk_elems)
            for r in range(n):
                assert np.array_equal(_bits(W.from_torch(recvs[r], dtype)), _bits(want[r])), (dtype, proto, r)


def test_ring_order_does_not_apply_to_the_tree():
    xs = W.inputs("tree-order", 6, 50001, "float32", "normal")
    a, _ = check(xs, "float32", "sum", "Simple", 3, 0)
    b, _ = check(xs, "float32", "sum", "Simple", 3, 0, ring_order=[3, 1, 5, 0, 2, 4])
    for x, y in zip(a, b):
        assert np.array_equal(_bits(x), _bits(y))

"""LL128 lane parts sized to reach each path of the line loop, bit-exact
against the oracle: whole 64-line row iterations only, iterations plus a
partly masked one, a part under one iteration, a part that is one line or
less, a ragged last line, a full 256-line slot and parts of two slices (a
flag round trip each).  The last line of every slice goes packet by packet
(its flag is the one stored after the slice's data).  Every dtype, ring (one
input) and tree (vertices with two inputs, where an iteration is 32 lines),
in place and out of place: in the whole rows lane 7 of a line moves data
bytes 104..119 and so shares 104..111 with lane 6, which the in-place cases
check.

With one channel and one lane, a ring part is one chunk, count / n
elements; its bytes are chosen as 120 x lines (+ a ragged tail) rounded to
whole 16-byte units.
"""
import numpy as np
import pytest
import torch

import oracle
import ring_allreduce_reduce_amd as ra
from ring_allreduce_reduce_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

# part bytes: (whole lines, ragged bytes) -> rounded up to 16-byte units
PARTS = [(64, 0), (65, 0), (128, 0), (100, 56), (63, 40), (20, 0), (17, 104), (140, 0), (192, 72), (256, 0),
         (9, 8), (300, 24), (1, 0), (0, 40), (257, 0), (33, 0)]


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


def _part_bytes(lines, tail):
    b = lines * 120 + tail
    return (b + 15) // 16 * 16


def _run(xs, dtype, op, algo, inplace):
    n = len(xs)
    count = xs[0].size
    sends = [W.to_torch(x, dtype, DEV) for x in xs]
    recvs = sends if inplace else [torch.zeros_like(s) for s in sends]
    cfg = dict(algo=algo, lanes=1)
    ra.allreduce(sends, recvs, op=op, nchannels=1, proto="LL128", **cfg)
    torch.cuda.synchronize()
    code = ra.ringar_get_async_error(torch.cuda.current_stream().cuda_stream)
    assert code == 0, ra.ringar_result_string(code)
    plan = ra.ringar_plan(count, dtype, n, 1, "LL128", ra.make_config(**cfg))
    run = oracle.tree_allreduce if plan.algo == 1 else oracle.ring_allreduce
    want = run(xs, dtype, op, plan.nchannels, plan.chunk_elems)
    return [W.from_torch(r, dtype) for r in recvs], want


@pytest.mark.parametrize("dtype", list(W.STORAGE))
@pytest.mark.parametrize("inplace", [False, True])
def test_ring_line_paths(dtype, inplace):
    es = W.ELEM_BYTES[dtype]
    for i, (lines, tail) in enumerate(PARTS):
        n = 3 if i % 2 else 2
        count = n * _part_bytes(lines, tail) // es
        op = ["sum", "max", "prod", "avg"][i % 4]
        dist = ("uniform", 0.9, 1.1) if (op == "prod" and dtype in W.FLOATS) else ("uniform", -4, 4)
        print(f"case LL128 ring {dtype} inplace={inplace} n={n} lines={lines}+{tail} count={count} {op}", flush=True)
        xs = W.inputs(f"ll128-lines-{dtype}-{i}", n, count, dtype, *dist)
        got, want = _run(xs, dtype, op, "ring", inplace)
        for r in range(n):
            assert np.array_equal(_bits(got[r]), _bits(want[r])), (dtype, inplace, lines, tail, r)


@pytest.mark.parametrize("dtype", ["int8", "bfloat16", "float32", "float64"])
@pytest.mark.parametrize("inplace", [False, True])
def test_tree_line_paths(dtype, inplace):
    # the tree's chunks follow its own size rule; several part sizes per n
    # still cover one- and two-input vertices over whole, masked and ragged
    # line runs
    es = W.ELEM_BYTES[dtype]
    for i, (lines, tail) in enumerate(PARTS):
        n = [5, 8, 6, 7][i % 4]
        count = 4 * _part_bytes(lines, tail) // es
        op = ["sum", "min", "avg"][i % 3]
        print(f"case LL128 tree {dtype} inplace={inplace} n={n} lines={lines}+{tail} count={count} {op}", flush=True)
        xs = W.inputs(f"ll128-tree-lines-{dtype}-{i}", n, count, dtype, "uniform", -4, 4)
        got, want = _run(xs, dtype, op, "tree", inplace)
        for r in range(n):
            assert np.array_equal(_bits(got[r]), _bits(want[r])), (dtype, inplace, n, lines, tail, r)

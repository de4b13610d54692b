"""Both block mappings against the oracle, bit for bit.

Which workgroup runs which (rank, channel, lane) changes only where the
wavefronts sit on MI355X's 8 XCDs, never what they compute.  Every
protocol, ring and tree, is run with the linear mapping and with the
XCD-major one (whose grid is padded to whole rounds of 8 groups, the padding
workgroups exiting at once) at sizes where the plan gives a single group,
group counts that are not multiples of 8, and the many groups of a large
call.
"""
import numpy as np
import pytest
import torch

import oracle
import ring_allreduce_reduce_amd as ra
from ring_allreduce_reduce_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

# (ranks, elements, channels, lanes): one group; 3 groups; 5 channels x 2
# lane blocks; 32 channels x 8 lanes (64 groups)
SHAPES = [(8, 2, 1, 0), (5, 3001, 3, 0), (7, 40000, 5, 8), (8, 1 << 20, 32, 8)]


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


@pytest.mark.parametrize("algo", ["ring", "tree"])
@pytest.mark.parametrize("proto", ["LL", "LL128", "Simple"])
@pytest.mark.parametrize("block_map", [1, 2])
def test_block_map_matches_oracle(algo, proto, block_map):
    for j, (n, count, nch, lanes) in enumerate(SHAPES):
        op = ["sum", "max", "avg", "prod"][j]
        dtype = ["float32", "bfloat16", "int32", "float16"][j]
        dist = ("uniform", 0.9, 1.1) if op == "prod" else ("uniform", -4, 4)
        cfg = dict(algo=algo, lanes=lanes, block_map=block_map)
        plan = ra.ringar_plan(count, dtype, n, nch, proto, ra.make_config(**cfg))
        assert plan.xcd_major == (block_map == 2)
        print(f"case {algo} {proto} block_map={block_map} n={n} count={count} nch={nch} lanes={plan.lanes} "
              f"grid={plan.workgroups} {dtype} {op}", flush=True)
        xs = W.inputs(f"blockmap-{algo}-{proto}-{j}", n, count, dtype, *dist)
        sends = [W.to_torch(x, dtype, DEV) for x in xs]
        recvs = [torch.zeros_like(s) for s in sends]
        ra.allreduce(sends, recvs, op=op, nchannels=nch, proto=proto, **cfg)
        torch.cuda.synchronize()
        code = ra.ringar_get_async_error(torch.cuda.current_stream().cuda_stream)
        assert code == 0, ra.ringar_result_string(code)
        run = oracle.tree_allreduce if plan.algo == 1 else oracle.ring_allreduce
        want = run(xs, dtype, op, plan.nchannels, plan.chunk_elems)
        for r in range(n):
            assert np.array_equal(_bits(W.from_torch(recvs[r], dtype)), _bits(want[r])), (algo, proto, j, r)


@pytest.mark.parametrize("n,nbytes", [(10, 1 << 19), (12, 1 << 18), (17, 1 << 18), (24, 1 << 19)])
def test_padding_beyond_residency_takes_the_linear_mapping(n, nbytes):
    # small enough for the XCD-major mapping by size, but its padded grid
    # would exceed the resident wavefronts: the plan takes the linear one,
    # and the automatic call runs (it used to be refused at launch)
    count = nbytes // 4
    cfg = dict(algo="auto")
    plan = ra.ringar_plan(count, "float32", n, 0, "auto", ra.make_config(**cfg))
    assert not plan.xcd_major
    print(f"case padding n={n} bytes={nbytes} algo={plan.algo} proto={plan.proto} nch={plan.nchannels} "
          f"lanes={plan.lanes} xcd_major={plan.xcd_major} grid={plan.workgroups}", flush=True)
    xs = W.inputs(f"blockmap-pad-{n}-{nbytes}", n, count, "float32", "uniform", -4, 4)
    sends = [W.to_torch(x, "float32", DEV) for x in xs]
    recvs = [torch.zeros_like(s) for s in sends]
    ra.allreduce(sends, recvs, op="sum", nchannels=0, proto="auto", **cfg)
    torch.cuda.synchronize()
    code = ra.ringar_get_async_error(torch.cuda.current_stream().cuda_stream)
    assert code == 0, ra.ringar_result_string(code)
    run = oracle.tree_allreduce if plan.algo == 1 else oracle.ring_allreduce
    want = run(xs, "float32", "sum", plan.nchannels, plan.chunk_elems)
    for r in range(n):
        assert np.array_equal(_bits(W.from_torch(recvs[r], "float32")), _bits(want[r])), r

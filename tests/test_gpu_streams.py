"""Calls on different streams use different FIFO memory and counters, so
they may run at the same time: several calls enqueued on two streams without
any synchronisation between them (small grids that fit on the GPU together),
ring and tree mixed, all equal the oracle."""
import numpy as np
import pytest
import torch

import oracle
import ring_allreduce_reduce_amd as ra
from ring_allreduce_reduce_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def test_two_streams_interleaved():
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    cases = []
    for j in range(8):
        n, count = (4, 30011) if j % 2 else (3, 77777)
        proto = ["LL", "Simple", "LL128"][j % 3]
        algo = "tree" if j % 4 == 3 else "ring"
        xs = W.inputs(f"streams-{j}", n, count, "float32", "normal")
        sends = [W.to_torch(x, "float32", DEV) for x in xs]
        recvs = [torch.zeros_like(s) for s in sends]
        cases.append((xs, sends, recvs, proto, algo, streams[j % 2]))
    torch.cuda.synchronize()
    for xs, sends, recvs, proto, algo, st in cases:
        # each stream waits for nothing but its own earlier calls
        ra.allreduce(sends, recvs, op="sum", nchannels=2, proto=proto, stream=st, algo=algo)
    torch.cuda.synchronize()
    for st in streams:
        assert ra.ringar_get_async_error(st.cuda_stream) == 0
    for xs, sends, recvs, proto, algo, st in cases:
        plan = ra.ringar_plan(xs[0].size, "float32", len(xs), 2, proto, ra.make_config(algo=algo))
        run = oracle.tree_allreduce if algo == "tree" else oracle.ring_allreduce
        want = run(xs, "float32", "sum", plan.nchannels, plan.chunk_elems)
        for r in range(len(xs)):
            assert np.array_equal(W.from_torch(recvs[r], "float32"), want[r]), (proto, algo, r)

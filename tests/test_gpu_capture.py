"""A call on a stream in graph capture is refused before anything is
enqueued (its FIFO step numbers would be replayed), and the library keeps
working afterwards."""
import numpy as np
import pytest
import torch

import oracle
import ring_allreduce_reduce_amd as ra
from ring_allreduce_reduce_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def test_capture_is_refused_and_later_calls_work():
    n, count = 4, 4096
    xs = W.inputs("capture", n, count, "float32", "normal")
    sends = [W.to_torch(x, "float32", DEV) for x in xs]
    recvs = [torch.zeros_like(s) for s in sends]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    codes = []
    with torch.cuda.graph(g):
        st = torch.cuda.current_stream().cuda_stream
        for algo in ("ring", "tree"):
            codes.append(ra.ringar_allreduce_ex([s.data_ptr() for s in sends], [r.data_ptr() for r in recvs],
                                                count, "float32", "sum", n, 2, "Simple", st,
                                                ra.make_config(algo=algo)))
    assert codes == [ra.INVALID_USAGE, ra.INVALID_USAGE]
    torch.cuda.synchronize()
    ra.allreduce(sends, recvs, op="sum", nchannels=2, proto="Simple")
    torch.cuda.synchronize()
    assert ra.ringar_get_async_error(torch.cuda.current_stream().cuda_stream) == 0
    plan = ra.ringar_plan(count, "float32", n, 2, "Simple")
    want = oracle.ring_allreduce(xs, "float32", "sum", plan.nchannels, plan.chunk_elems)
    for r in range(n):
        assert np.array_equal(W.from_torch(recvs[r], "float32"), want[r])

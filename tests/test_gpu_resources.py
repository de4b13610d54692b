"""Resource and capacity paths on the GPU: a grid larger than the GPU can
hold at once is refused before launch (its wavefronts wait on each other, so
all must be resident); ringar_release frees every FIFO and counter and the
next calls rebuild them and still match the oracle."""
import numpy as np
import pytest
import torch

import oracle
import ring_allreduce_reduce_amd as ra
from ring_allreduce_reduce_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _check(xs, proto, nch, algo="ring"):
    sends = [W.to_torch(x, "float32", DEV) for x in xs]
    recvs = [torch.zeros_like(s) for s in sends]
    ra.allreduce(sends, recvs, op="sum", nchannels=nch, proto=proto, algo=algo)
    torch.cuda.synchronize()
    assert ra.ringar_get_async_error(torch.cuda.current_stream().cuda_stream) == 0
    plan = ra.ringar_plan(xs[0].size, "float32", len(xs), nch, proto, ra.make_config(algo=algo))
    run = oracle.tree_allreduce if algo == "tree" else oracle.ring_allreduce
    want = run(xs, "float32", "sum", plan.nchannels, plan.chunk_elems)
    for r in range(len(xs)):
        assert np.array_equal(W.from_torch(recvs[r], "float32"), want[r])


def test_grid_beyond_residency_is_refused():
    n, count = 64, 1 << 20
    sends = [torch.zeros(count, device=DEV) for _ in range(n)]
    recvs = [torch.zeros(count, device=DEV) for _ in range(n)]
    st = torch.cuda.current_stream().cuda_stream
    # 64 ranks x 64 channels x 32 lanes = 131072 wavefronts: far more than the GPU holds
    cfg = ra.make_config(lanes=32)
    code = ra.ringar_allreduce_ex([s.data_ptr() for s in sends], [r.data_ptr() for r in recvs], count,
                                  "float32", "sum", n, 64, "Simple", st, cfg)
    assert code == ra.INVALID_USAGE
    code = ra.ringar_allreduce_ex([s.data_ptr() for s in sends], [r.data_ptr() for r in recvs], count,
                                  "float32", "sum", n, 64, "Simple", st, ra.make_config(lanes=32, algo="tree"))
    assert code == ra.INVALID_USAGE
    torch.cuda.synchronize()
    assert ra.ringar_get_async_error(st) == 0
    # nothing was enqueued: the outputs are untouched
    assert all(int(torch.count_nonzero(r)) == 0 for r in recvs[:4])


def test_release_then_calls_rebuild_their_resources():
    xs = W.inputs("release", 6, 123457, "float32", "normal")
    for proto in ("LL", "LL128", "Simple"):
        _check(xs, proto, 3)
    ra.ringar_release()
    for proto in ("Simple", "LL", "LL128"):
        _check(xs, proto, 3)
        _check(xs, proto, 3, algo="tree")
    ra.ringar_release()
    _check(xs, "Simple", 2)

"""Parity of the average (sum folded, divided by n once where a value becomes
final) on the GPU with the CPU oracle, bit for bit: the ring under all three
protocols in both kernel forms and the direct form, the tree, and the
ReduceScatter half, every dtype, ragged shapes and several rank counts."""
import numpy as np
import pytest
import torch

import oracle
import ring_allreduce_reduce_amd as ra
from ring_allreduce_reduce_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
DTYPES = list(W.STORAGE)
SHAPES = [(2, 1, 1), (3, 1001, 2), (8, 65537, 4), (5, 300007, 3), (8, 1 << 20, 16)]


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


def _sync_ok():
    torch.cuda.synchronize()
    code = ra.ringar_get_async_error(torch.cuda.current_stream().cuda_stream)
    assert code == 0, ra.ringar_result_string(code)


@pytest.mark.parametrize("variant", ["LL", "LL128", "Simple", "Simple-general", "direct", "tree-LL", "tree-LL128",
                                     "tree-Simple"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_allreduce_average(variant, dtype):
    proto = variant.split("-")[-1] if variant != "direct" else "Simple"
    if proto == "general":
        proto = "Simple"
    algo = "tree" if variant.startswith("tree") else "ring"
    for i, (n, count, nch) in enumerate(SHAPES):
        print(f"case avg {variant} {dtype} n={n} count={count} nch={nch}", flush=True)
        xs = W.inputs(f"gavg-{dtype}-{i}", n, count, dtype, "uniform", -4, 4)
        sends = [W.to_torch(x, dtype, DEV) for x in xs]
        recvs = [torch.zeros_like(t) for t in sends]
        kw = dict(algo=algo, direct=int(variant == "direct"), force_general=int(variant == "Simple-general"))
        ra.allreduce(sends, recvs, op="avg", nchannels=nch, proto=proto, **kw)
        _sync_ok()
        plan = ra.ringar_plan(count, dtype, n, nch, proto, ra.make_config(**kw))
        run = oracle.tree_allreduce if plan.algo == 1 else oracle.ring_allreduce
        want = run(xs, dtype, "avg", plan.nchannels, plan.chunk_elems)
        for r in range(n):
            assert np.array_equal(_bits(W.from_torch(recvs[r], dtype)), _bits(want[r])), (variant, dtype, n, r)


@pytest.mark.parametrize("proto", ["LL", "LL128", "Simple"])
@pytest.mark.parametrize("dtype", DTYPES)
def test_reduce_scatter_average(proto, dtype):
    for i, (n, count, nch) in enumerate(SHAPES[:4]):
        print(f"case avg reduce_scatter {proto} {dtype} n={n} count={count}", flush=True)
        xs = W.inputs(f"gavg-rs-{dtype}-{i}", n, n * count, dtype, "uniform", -4, 4)
        sends = [W.to_torch(x, dtype, DEV) for x in xs]
        recvs = [torch.zeros(count, dtype=sends[0].dtype, device=DEV) for _ in range(n)]
        ra.reduce_scatter(sends, recvs, op="avg", nchannels=nch, proto=proto)
        _sync_ok()
        want = oracle.ring_reduce_scatter(xs, dtype, "avg")
        for r in range(n):
            assert np.array_equal(_bits(W.from_torch(recvs[r], dtype)), _bits(want[r])), (proto, dtype, n, r)

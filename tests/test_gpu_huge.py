"""Buffers beyond 4 GiB per rank (more than 2^32 bytes and elements): int8
sum over 8 ranks of 4.5 Gi + 13 elements, every rank zero except three
marked elements (the first, one just past 2^32, the last), so the exact
result is known in closed form (the pages' worked example, extended): the
first element is 0+1+...+7 = 28, the one past 2^32 is 8, the last is
1+2+...+8 = 36, everything else 0.  Checked on the GPU for the ring under
Simple and LL and for the tree."""
import pytest
import torch

import ring_allreduce_reduce_amd as ra

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
COUNT = (9 << 29) + 13          # 4.5 Gi + 13 elements
MID = (1 << 32) + 5


@pytest.fixture(scope="module")
def buffers():
    sends = []
    for r in range(8):
        x = torch.zeros(COUNT, dtype=torch.int8, device=DEV)
        x[0] = r
        x[MID] = 1
        x[COUNT - 1] = r + 1
        sends.append(x)
    recvs = [torch.empty_like(s) for s in sends]
    yield sends, recvs
    del sends, recvs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("proto,algo", [("Simple", "ring"), ("LL", "ring"), ("Simple", "tree")])
def test_beyond_4GiB_per_rank(buffers, proto, algo):
    sends, recvs = buffers
    print(f"case huge {proto} {algo} count={COUNT}", flush=True)
    for r in recvs:
        r.fill_(-1)
    ra.allreduce(sends, recvs, op="sum", proto=proto, algo=algo)
    torch.cuda.synchronize()
    assert ra.ringar_get_async_error(torch.cuda.current_stream().cuda_stream) == 0
    for r in range(8):
        y = recvs[r]
        assert int(y[0]) == 28 and int(y[MID]) == 8 and int(y[COUNT - 1]) == 36, (proto, algo, r)
        assert int(torch.count_nonzero(y)) == 3, (proto, algo, r)

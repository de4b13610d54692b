"""Every call whose knobs are left to the library runs.

A grid of rank counts (2..64), sizes (8 B .. 64 MiB per rank), dtypes,
algorithms, protocols and channel counts (automatic or forced), with no
other knob forced: each call must be accepted (no refusal at planning or
at launch, such as a grid beyond residency) and end without an
asynchronous error; the AllReduce of all-ones inputs is checked after each
group of calls (every output element equals n).  Parity of the values is
the other tests' job; this one guards the plan's rules against refusing
what they should run.
"""
import pytest
import torch

import ring_allreduce_reduce_amd as ra

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
RANKS = [2, 3, 5, 8, 10, 12, 16, 17, 24, 33, 64]
SIZES = [8, 1024, 32768, 262144, 524288, 1 << 20, 4 << 20]


@pytest.mark.parametrize("n", RANKS)
def test_every_automatic_call_runs(n):
    sizes = SIZES + ([64 << 20] if n <= 16 else [])
    stream = torch.cuda.current_stream().cuda_stream
    for nbytes in sizes:
        for dtype in (torch.float32, torch.int8):
            es = torch.tensor([], dtype=dtype).element_size()
            count = max(1, nbytes // es)
            print(f"case accept n={n} bytes={nbytes} {dtype}", flush=True)
            xs = [torch.ones(count, device=DEV, dtype=dtype) for _ in range(n)]
            ys = [torch.zeros_like(x) for x in xs]
            for algo in ("auto", "ring", "tree"):
                for proto in ("auto", "LL", "LL128", "Simple"):
                    for nch in (0, 1, 3, 13, 32):
                        ra.allreduce(xs, ys, op="sum", nchannels=nch, proto=proto, algo=algo)
            torch.cuda.synchronize()
            code = ra.ringar_get_async_error(stream)
            assert code == 0, (n, nbytes, dtype, ra.ringar_result_string(code))
            for y in ys:
                assert bool((y == n).all()), (n, nbytes, dtype)

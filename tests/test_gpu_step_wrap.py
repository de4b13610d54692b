"""The step numbers restart before the 32-bit LL flags would wrap: all FIFO
memory and counters are cleared and numbering starts again at zero.  The
stream's step base is started just below that point (test hook
RINGAR_STEP_BASE, read when a stream's resources are created), so a few
hundred small calls of every protocol and both algorithms cross it; every
call equals the oracle."""
import os

import numpy as np
import pytest
import torch

import oracle
import ring_allreduce_reduce_amd as ra
from ring_allreduce_reduce_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
RESTART = 0xFFFFFFF0


def test_calls_across_the_restart():
    start = RESTART - 3000
    os.environ["RINGAR_STEP_BASE"] = str(start)
    try:
        st = torch.cuda.Stream()          # new resources pick up the hook
        xs = W.inputs("wrap", 8, 5003, "float32", "normal")
        sends = [W.to_torch(x, "float32", DEV) for x in xs]
        recvs = [torch.zeros_like(s) for s in sends]
        torch.cuda.synchronize()
        base, crossed, calls = start, False, 0
        wants = {}
        while calls < 400 and not (crossed and calls > 60):
            proto = ["LL", "LL128", "Simple"][calls % 3]
            algo = "tree" if calls % 5 == 4 else "ring"
            cfg = ra.make_config(algo=algo)
            plan = ra.ringar_plan(5003, "float32", 8, 2, proto, cfg)
            if base + plan.max_steps + 1 >= RESTART:
                crossed = True
                base = 0
            with torch.cuda.stream(st):       # cleared on the call's own stream
                for r in recvs:
                    r.zero_()
            ra.allreduce(sends, recvs, op="sum", nchannels=2, proto=proto, stream=st, algo=algo)
            st.synchronize()
            assert ra.ringar_get_async_error(st.cuda_stream) == 0, (calls, proto, algo)
            key = (algo, plan.nchannels, plan.chunk_elems)
            if key not in wants:
                run = oracle.tree_allreduce if algo == "tree" else oracle.ring_allreduce
                wants[key] = run(xs, "float32", "sum", plan.nchannels, plan.chunk_elems)
            for r in range(8):
                assert np.array_equal(W.from_torch(recvs[r], "float32"), wants[key][r]), (calls, proto, algo, r, base)
            base += plan.max_steps + 1
            calls += 1
        assert crossed, "the calls did not reach the restart"
    finally:
        del os.environ["RINGAR_STEP_BASE"]

"""Parity with the CPU oracle, bit for bit, over randomly drawn calls.

Each case draws every knob of a call at once: rank count (1 to 64), element
count (0 to about a million, log-uniform), dtype, op, protocol, algorithm,
direct form, channels, chunk, lanes, FIFO depth, ring order, in-place or
out-of-place, 16-byte-misaligned buffers, the elementwise kernel form and
the block mapping (linear or XCD-major).
The fixed tests cover each knob on its own; these cover their combinations.
A request whose plan the library refuses (a forced lane count or mapping
whose grid is beyond residency, a forced lane count the FIFO budget cannot
hold) is skipped and counted, and the test asserts most cases ran; a call
whose plan was made must run.  The oracle runs with the plan's
resolved channels and chunk, and the tree ignores the ring order as the
library does.
"""
import numpy as np
import pytest
import torch

import oracle
import ring_allreduce_reduce_amd as ra
from ring_allreduce_reduce_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
DTYPES = list(W.STORAGE)
OPS = ["sum", "prod", "min", "max", "avg"]
CASES = 150


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


def _draw(rng, halves=False):
    n = int(rng.integers(2, 17)) if rng.random() < 0.8 else int(rng.integers(17, 65))
    if rng.random() < 0.03:
        n = 1
    count = int(np.exp(rng.uniform(0, np.log(1_000_000 if n <= 16 else 100_000))))
    if halves:
        count = max(count // n, 0)
    if rng.random() < 0.03:
        count = 0
    dtype = DTYPES[int(rng.integers(0, len(DTYPES)))]
    op = OPS[int(rng.integers(0, len(OPS)))]
    proto = ["LL", "LL128", "Simple", "auto"][int(rng.integers(0, 4))]
    chunk = 0 if rng.random() < 0.5 else int(rng.integers(1, 4096)) * 16
    cfg = dict(chunk_bytes=chunk,
               lanes=0 if rng.random() < 0.6 else int(2 ** rng.integers(0, 6)),
               fifo_depth=0 if rng.random() < 0.7 else int([2, 4, 8][rng.integers(0, 3)]),
               force_general=int(rng.random() < 0.2),
               ring_order=[int(r) for r in rng.permutation(n)] if rng.random() < 0.3 else None)
    if not halves:
        cfg["algo"] = ["ring", "tree", "auto"][int(rng.integers(0, 3))]
        cfg["direct"] = int(rng.random() < 0.3)
    nch = int(rng.integers(0, 17))
    inplace = rng.random() < 0.2
    unaligned = (not inplace) and rng.random() < 0.15
    # block mapping: by size, or either mapping forced at any size
    cfg["block_map"] = int(rng.integers(0, 3))
    return n, count, dtype, op, proto, nch, cfg, inplace, unaligned


def _tensors(xs, dtype, count, recv_count, unaligned):
    if not unaligned:
        return [W.to_torch(x, dtype, DEV) for x in xs], None
    sends = [W.to_torch(np.concatenate([np.zeros(1, x.dtype), x]), dtype, DEV)[1:] for x in xs]
    recvs = [torch.zeros(recv_count + 1, dtype=sends[0].dtype, device=DEV)[1:] for _ in xs]
    return sends, recvs


def _dist(op, dtype):
    # products of many ranks stay finite and far from rounding ties near 1
    return ("uniform", 0.9, 1.1) if (op == "prod" and dtype in W.FLOATS) else ("uniform", -4, 4)


def _finish():
    torch.cuda.synchronize()
    return ra.ringar_get_async_error(torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("seed", [101, 202, 303])
def test_random_allreduce(seed):
    rng = np.random.default_rng(seed)
    ran = skipped = 0
    for i in range(CASES):
        n, count, dtype, op, proto, nch, cfg, inplace, unaligned = _draw(rng)
        try:
            plan = ra.ringar_plan(count, dtype, n, nch, proto, ra.make_config(**cfg))
        except ra.RingarError:
            skipped += 1
            continue
        desc = (f"allreduce seed {seed} case {i}: n={n} count={count} {dtype} {op} {proto} nch={nch} {cfg} "
                f"inplace={inplace} unaligned={unaligned} -> {ra.ALGO_NAMES[plan.algo]} "
                f"{ra.PROTO_NAMES[plan.proto]} ch={plan.nchannels} lanes={plan.lanes} depth={plan.fifo_depth}")
        print(desc, flush=True)
        xs = W.inputs(f"grand-{seed}-{i}", n, count, dtype, *_dist(op, dtype))
        sends, recvs = _tensors(xs, dtype, count, count, unaligned)
        if recvs is None:
            recvs = sends if inplace else [torch.zeros_like(t) for t in sends]
        # a call whose plan was made runs: the plan refuses what the launch
        # would (a forced lane count or mapping beyond residency)
        ra.allreduce(sends, recvs, op=op, nchannels=nch, proto=proto, **cfg)
        code = _finish()
        assert code == 0, (desc, ra.ringar_result_string(code))
        if plan.algo == 1:
            want = oracle.tree_allreduce(xs, dtype, op, plan.nchannels, plan.chunk_elems)
        else:
            want = oracle.ring_allreduce(xs, dtype, op, plan.nchannels, plan.chunk_elems, ring=cfg["ring_order"])
        for r in range(n):
            assert np.array_equal(_bits(W.from_torch(recvs[r], dtype)), _bits(want[r])), (desc, r)
        ran += 1
    assert ran >= CASES * 3 // 4, (ran, skipped)


@pytest.mark.parametrize("coll", ["reduce_scatter", "all_gather"])
def test_random_halves(coll):
    rng = np.random.default_rng(404 if coll == "reduce_scatter" else 505)
    ran = skipped = 0
    for i in range(CASES):
        n, count, dtype, op, proto, nch, cfg, inplace, unaligned = _draw(rng, halves=True)
        try:
            ra.ringar_plan_coll(coll, count, dtype, n, nch, proto, ra.make_config(**cfg))
        except ra.RingarError:
            skipped += 1
            continue
        desc = (f"{coll} case {i}: n={n} count={count} {dtype} {op} {proto} nch={nch} {cfg} "
                f"inplace={inplace} unaligned={unaligned}")
        print(desc, flush=True)
        rs = coll == "reduce_scatter"
        send_count, recv_count = (n * count, count) if rs else (count, n * count)
        xs = W.inputs(f"grand-{coll}-{i}", n, send_count, dtype, *_dist(op, dtype))
        sends, recvs = _tensors(xs, dtype, send_count, recv_count, unaligned)
        if recvs is None:
            if inplace and rs:
                # the pages' in-place ReduceScatter: rank r's result is block r of its own buffer
                recvs = [t[r * count:(r + 1) * count] for r, t in enumerate(sends)]
            elif inplace:
                full = [torch.zeros(n * count, dtype=sends[0].dtype, device=DEV) for _ in range(n)]
                for r in range(n):
                    full[r][r * count:(r + 1) * count].copy_(sends[r])
                sends = [full[r][r * count:(r + 1) * count] for r in range(n)]
                recvs = full
            else:
                recvs = [torch.zeros(recv_count, dtype=sends[0].dtype, device=DEV) for _ in range(n)]
        if rs:
            ra.reduce_scatter(sends, recvs, op=op, nchannels=nch, proto=proto, **cfg)
        else:
            ra.all_gather(sends, recvs, nchannels=nch, proto=proto, **cfg)
        code = _finish()
        assert code == 0, (desc, ra.ringar_result_string(code))
        if rs:
            want = oracle.ring_reduce_scatter(xs, dtype, op, ring=cfg["ring_order"])
        else:
            want = oracle.ring_all_gather(xs, dtype, ring=cfg["ring_order"])
        for r in range(n):
            assert np.array_equal(_bits(W.from_torch(recvs[r], dtype)), _bits(want[r])), (desc, r)
        ran += 1
    assert ran >= CASES * 3 // 4, (ran, skipped)


def test_random_split_tree():
    """Random calls that the tree runs in its split form (eager Simple, at
    least 256 KiB per channel), every other knob drawn as above."""
    rng = np.random.default_rng(606)
    ran = split = 0
    for i in range(40):
        n = int(rng.integers(2, 17)) if rng.random() < 0.9 else int(rng.integers(17, 33))
        dtype = DTYPES[int(rng.integers(0, len(DTYPES)))]
        es = W.ELEM_BYTES[dtype]
        op = OPS[int(rng.integers(0, len(OPS)))]
        nch = int(rng.integers(1, 9))
        count = int(rng.integers((256 << 10) * nch // es, (1 << 20) * nch // es + 1)) + int(rng.integers(0, 17))
        cfg = dict(algo="tree",
                   chunk_bytes=0 if rng.random() < 0.5 else int(rng.integers(64, 16384)) * 16,
                   lanes=0 if rng.random() < 0.7 else int(2 ** rng.integers(0, 4)),
                   fifo_depth=0 if rng.random() < 0.7 else int([2, 4, 8][rng.integers(0, 3)]),
                   block_map=int(rng.integers(0, 3)))
        inplace = rng.random() < 0.2
        unaligned = (not inplace) and rng.random() < 0.15
        try:
            plan = ra.ringar_plan(count, dtype, n, nch, "Simple", ra.make_config(**cfg))
        except ra.RingarError:
            continue
        desc = (f"split tree case {i}: n={n} count={count} {dtype} {op} nch={nch} {cfg} inplace={inplace} "
                f"unaligned={unaligned} -> split={plan.tree_split} lanes={plan.lanes} depth={plan.fifo_depth} "
                f"chunk={plan.chunk_elems * es}")
        print(desc, flush=True)
        xs = W.inputs(f"grand-split-{i}", n, count, dtype, *_dist(op, dtype))
        sends, recvs = _tensors(xs, dtype, count, count, unaligned)
        if recvs is None:
            recvs = sends if inplace else [torch.zeros_like(t) for t in sends]
        ra.allreduce(sends, recvs, op=op, nchannels=nch, proto="Simple", **cfg)
        code = _finish()
        assert code == 0, (desc, ra.ringar_result_string(code))
        want = oracle.tree_allreduce(xs, dtype, op, plan.nchannels, plan.chunk_elems)
        for r in range(n):
            assert np.array_equal(_bits(W.from_torch(recvs[r], dtype)), _bits(want[r])), (desc, r)
        ran += 1
        split += plan.tree_split
    assert ran >= 28 and split >= ran * 3 // 4, (ran, split)

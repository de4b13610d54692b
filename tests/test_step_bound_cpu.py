"""The step bound of a plan covers every connection (CPU only).

Each call advances the stream's step base by max_steps + 1, and stale
counters and flags of a call are only safe because no connection of that
call takes more than max_steps steps.  This test replays the partition of
random plans (the oracle's channel and loop rules, the plan's chunk, lanes
and protocol) and counts the FIFO slices every connection carries: one per
started slot of each non-empty lane part the connection moves.
"""
import numpy as np
import pytest

import oracle
import ring_allreduce_reduce_amd as ra
from libutil import lib

SLOT_DATA = {"Simple": 32768, "LL": 8192, "LL128": 30720}
# lane parts are whole multiples of this many bytes: 1 KiB, and 8 lines of
# 120 data bytes under LL128 (so a part ends on a whole line)
LANE_GRAN = {"Simple": 1024, "LL": 1024, "LL128": 960}
ES = {"int8": 1, "int32": 4, "float16": 2, "bfloat16": 2, "float32": 4, "float64": 8}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    lib()


def _lane_parts(clen, cur, lanes, es, proto):
    part = -(-cur // lanes)
    g = LANE_GRAN[proto] // es
    part = -(-part // g) * g
    out = []
    for l in range(lanes):
        s = min(clen, l * part)
        out.append(min(clen, s + part) - s)
    return out


def _slices(nelem, es, proto):
    return -(-(nelem * es) // SLOT_DATA[proto]) if nelem else 0


def _loop_slices(rem, cur, n, lanes, es, proto):
    """Slices per lane of one ring loop with `rem` elements left and chunk
    size `cur` (chunk k = [k cur, min(rem, (k + 1) cur)))."""
    per_lane = np.zeros(lanes, dtype=np.int64)
    for k in range(n):
        ks = min(rem, k * cur)
        kl = min(cur, rem - ks) if ks < rem else 0
        for l, ll in enumerate(_lane_parts(kl, cur, lanes, es, proto)):
            per_lane[l] += _slices(ll, es, proto)
    return per_lane


def ring_steps(count, dtype, n, plan, proto):
    """An upper bound of the slices any ring connection carries: per loop a
    connection moves each chunk of the loop at most twice (2n - 2 sends over
    n chunks)."""
    es = ES[dtype]
    worst = 0
    for c in range(plan.nchannels):
        lo, hi = oracle.channel_range(count, dtype, plan.nchannels, c)
        length = hi - lo
        loop = n * plan.chunk_elems
        full = length // loop
        per_lane = full * _loop_slices(loop, plan.chunk_elems, n, plan.lanes, es, proto)
        if length > full * loop:
            off = full * loop
            cur = oracle.loop_chunk(length, off, dtype, n, plan.chunk_elems)
            per_lane = per_lane + _loop_slices(length - off, cur, n, plan.lanes, es, proto)
        worst = max(worst, int(per_lane.max()))
    return 2 * worst


def blocked_steps(count, dtype, plan, proto, primitives_per_chunk):
    """Halves and tree: loops take chunk_elems of the channel (of a block)."""
    es = ES[dtype]
    worst = 0
    for c in range(plan.nchannels):
        lo, hi = oracle.channel_range(count, dtype, plan.nchannels, c)
        length = hi - lo
        full = length // plan.chunk_elems
        per_lane = full * np.array([_slices(ll, es, proto) for ll in
                                    _lane_parts(plan.chunk_elems, plan.chunk_elems, plan.lanes, es, proto)], dtype=np.int64)
        tail = length - full * plan.chunk_elems
        if tail:
            per_lane = per_lane + np.array([_slices(ll, es, proto) for ll in
                                            _lane_parts(tail, tail, plan.lanes, es, proto)], dtype=np.int64)
        worst = max(worst, int(per_lane.max()))
    return worst * primitives_per_chunk


CASES = []
rng = np.random.default_rng(2024)
for i in range(300):
    CASES.append((int(rng.integers(2, 17)), int(rng.integers(1, 3_000_000)), int(rng.integers(0, 33)),
                  ["LL", "LL128", "Simple"][i % 3], list(ES)[int(rng.integers(0, 6))],
                  int(rng.choice([0, 0, 1, 3, 17, 64])) * 16))


@pytest.mark.parametrize("case", range(0, 300, 30))
def test_ring_allreduce_step_bound(case):
    for n, count, nch, proto, dtype, chunk in CASES[case:case + 30]:
        cfg = ra.make_config(chunk_bytes=chunk)
        try:
            p = ra.ringar_plan(count, dtype, n, nch, proto, cfg)
        except ra.RingarError:
            continue
        steps = ring_steps(count, dtype, n, p, proto)
        assert steps <= p.max_steps, (n, count, nch, proto, dtype, chunk, steps, p.max_steps)
        d = ra.ringar_plan(count, dtype, n, nch, "Simple", ra.make_config(chunk_bytes=chunk, direct=1))
        assert ring_steps(count, dtype, n, d, "Simple") <= d.max_steps


@pytest.mark.parametrize("case", range(0, 300, 30))
def test_tree_step_bound(case):
    for n, count, nch, proto, dtype, chunk in CASES[case:case + 30]:
        try:
            p = ra.ringar_plan(count, dtype, n, nch, proto, ra.make_config(chunk_bytes=chunk, algo="tree"))
        except ra.RingarError:
            continue
        assert p.algo == 1
        assert blocked_steps(count, dtype, p, proto, 1) <= p.max_steps, (n, count, nch, proto, dtype, chunk)


@pytest.mark.parametrize("case", range(0, 300, 30))
def test_halves_step_bound(case):
    for n, count, nch, proto, dtype, chunk in CASES[case:case + 30]:
        block = max(1, count // n)
        for coll in ("reduce_scatter", "all_gather"):
            try:
                p = ra.ringar_plan_coll(coll, block, dtype, n, nch, proto, ra.make_config(chunk_bytes=chunk))
            except ra.RingarError:
                continue
            kdtype = "int8" if coll == "all_gather" else dtype
            kcount = block * ES[dtype] if coll == "all_gather" else block
            # a loop takes one chunk of every block; each connection carries n - 1 of them
            assert blocked_steps(kcount, kdtype, p, proto, n) <= p.max_steps, (coll, n, block, nch, proto, dtype)

"""The C-ABI library on the CPU: it loads, exports what include/ringar.h
declares, and its host logic (plan, protocol model, partition, argument
checks) agrees with the oracle.  No call here reaches the GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import ring_allreduce_reduce_amd as ra
from libutil import golden_model_dict, lib, lib_model, oracle_model
from oracle import select as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _lib():
    lib()
    os.environ.pop("RINGAR_PROTO", None)


def test_exports_every_declared_symbol():
    with open(os.path.join(ROOT, "include", "ringar.h")) as f:
        text = f.read()
    names = set(re.findall(r"^\s*(?:ringar_result_t|const char\*)\s+(ringar_\w+)\s*\(", text, re.M))
    assert "ringar_allreduce" in names and len(names) >= 10
    cdll = ctypes.CDLL(ra.LIB_PATH)
    for name in sorted(names):
        assert hasattr(cdll, name), name


def test_default_model_is_the_documented_one():
    m = ra.ringar_default_model()
    d = golden_model_dict()
    assert m.bw_per_channel == d["bw_per_channel"]
    assert m.ll_max_bw == d["ll_max_bw"]
    assert m.ll128_per_channel_max_bw == d["ll128_per_channel_max_bw"]
    assert list(m.eff) == d["eff"]
    assert list(m.base_lat_us) == d["base_lat_us"]
    assert list(m.hw_lat_us) == d["hw_lat_us"]
    assert (m.max_channels, m.max_pairs) == (d["max_channels"], d["max_pairs"])
    assert list(m.threads) == d["threads"]
    assert list(m.thread_threshold) == d["thread_threshold"]
    assert list(m.default_chunk_bytes) == d["default_chunk_bytes"]


def test_select_matches_oracle_model_and_pages_table():
    # the pages' 8x A100 inputs through the library's selector
    d = dict(golden_model_dict(), bw_per_channel=20.0, ll_max_bw=87.7, ll128_per_channel_max_bw=36.7,
             eff=[0.5, 0.92, 1.0], base_lat_us=[6.6, 14.0, 8.4], hw_lat_us=[0.6, 1.9, 3.4])
    m, om = lib_model(d), oracle_model(d)
    for nbytes in [8, 1000, 1 << 16, 1 << 20, 3 << 22, 1 << 26, 1 << 30]:
        p, t = ra.ringar_select(nbytes, 8, 24, m)
        op, ot = S.select(om, 8, 24, nbytes)
        assert p == op
        assert np.allclose(t, ot, rtol=1e-12, atol=0)
    _, t = ra.ringar_select(0, 8, 24, m)
    assert t[2] == pytest.approx(56.0, abs=0.05) and t[1] == pytest.approx(40.6, abs=0.05)


PLAN_CASES = [(b, n, nch, proto)
              for b in [8, 64, 1000, 4096, 65536, 1 << 20, 5 << 20, 64 << 20, 1 << 30]
              for n in [2, 3, 8]
              for nch in [0, 1, 16]
              for proto in ["auto", "LL", "LL128", "Simple"]]


@pytest.mark.parametrize("dtype", ["int8", "float32", "float64"])
def test_plan_matches_oracle_resolution(dtype):
    om = oracle_model()
    es = ra.ELEM_BYTES[dtype]
    for nbytes, n, nch, proto in PLAN_CASES:
        count = nbytes // es
        plan = ra.ringar_plan(count, dtype, n, nch, proto)
        want = S.resolve(om, n, count * es, nch, None if proto == "auto" else proto)
        assert (ra.PROTO_NAMES[plan.proto], plan.nchannels, plan.chunk_bytes) == want, (nbytes, n, nch, proto)
        assert plan.chunk_elems * es == plan.chunk_bytes
        assert plan.channel_elems == oracle.channel_range(count, dtype, plan.nchannels, 0)[1] or count == 0 \
            or plan.channel_elems >= count


def test_partition_matches_oracle():
    rng = np.random.default_rng(5)
    for _ in range(60):
        dtype = ["int8", "int32", "float16", "bfloat16", "float32", "float64"][int(rng.integers(0, 6))]
        es = ra.ELEM_BYTES[dtype]
        n = int(rng.integers(2, 9))
        nch = int(rng.integers(1, 6))
        chunk = int(rng.integers(1, 5)) * (16 // es)
        count = int(rng.integers(0, 3000))
        want = oracle.element_chunks(count, dtype, n, nch, chunk)
        got = np.full(count, -1, dtype=np.int32)
        for c in range(nch):
            lo, hi, _, _ = ra.ringar_chunk_range(count, dtype, n, nch, chunk, c, 0, 0)
            assert (lo, hi) == oracle.channel_range(count, dtype, nch, c)
            off = 0
            while off < hi - lo:
                for k in range(n):
                    _, _, klo, khi = ra.ringar_chunk_range(count, dtype, n, nch, chunk, c, off, k)
                    got[klo:khi] = k
                off += n * chunk
        assert np.array_equal(got, want)


def _fake(n, step=1 << 20, base=1 << 32):
    return [base + i * step for i in range(n)]


def test_argument_errors_before_any_device_call():
    n, count = 4, 1000
    s, r = _fake(n), _fake(n, base=1 << 40)
    E = ra
    assert ra.ringar_allreduce(s, r, count, 9, "sum", n, 2, "Simple", 0) == E.INVALID_ARGUMENT
    assert ra.ringar_allreduce(s, r, count, "float32", 7, n, 2, "Simple", 0) == E.INVALID_ARGUMENT
    assert ra.ringar_allreduce(s, r, count, "float32", "sum", n, 2, 5, 0) == E.INVALID_ARGUMENT
    assert ra.ringar_allreduce(s, r, count, "float32", "sum", 0, 2, "Simple", 0) == E.INVALID_ARGUMENT
    assert ra.ringar_allreduce(s, r, count, "float32", "sum", 65, 2, "Simple", 0) == E.INVALID_ARGUMENT
    assert ra.ringar_allreduce(s, r, count, "float32", "sum", n, 65, "Simple", 0) == E.INVALID_ARGUMENT
    assert ra.ringar_allreduce(s, r, count, "float32", "sum", n, -1, "Simple", 0) == E.INVALID_ARGUMENT
    bad_chunk = ra.make_config(chunk_bytes=24)
    assert ra.ringar_allreduce_ex(s, r, count, "float32", "sum", n, 2, "Simple", 0, bad_chunk) == E.INVALID_ARGUMENT
    bad_ring = ra.make_config(ring_order=[0, 1, 1, 3])
    assert ra.ringar_allreduce_ex(s, r, count, "float32", "sum", n, 2, "Simple", 0, bad_ring) == E.INVALID_ARGUMENT
    bad_lanes = ra.make_config(lanes=3)
    assert ra.ringar_allreduce_ex(s, r, count, "float32", "sum", n, 2, "Simple", 0, bad_lanes) == E.INVALID_ARGUMENT
    # misaligned pointer
    s2 = list(s)
    s2[1] += 2
    assert ra.ringar_allreduce(s2, r, count, "float32", "sum", n, 2, "Simple", 0) == E.INVALID_ARGUMENT
    # null pointer with work to do
    assert ra.ringar_allreduce([0] * n, r, count, "float32", "sum", n, 2, "Simple", 0) == E.INVALID_ARGUMENT
    # overlaps: receive buffers of two ranks, receive with another rank's send
    r2 = list(r)
    r2[2] = r2[1] + 400
    assert ra.ringar_allreduce(s, r2, count, "float32", "sum", n, 2, "Simple", 0) == E.INVALID_USAGE
    r3 = list(r)
    r3[0] = s[3]
    assert ra.ringar_allreduce(s, r3, count, "float32", "sum", n, 2, "Simple", 0) == E.INVALID_USAGE
    r4 = list(r)
    r4[1] = s[1] + 4          # partial in-place overlap
    assert ra.ringar_allreduce(s, r4, count, "float32", "sum", n, 2, "Simple", 0) == E.INVALID_USAGE
    # count == 0 succeeds without touching anything
    assert ra.ringar_allreduce(s, r, 0, "float32", "sum", n, 2, "Simple", 0) == E.SUCCESS


def test_proto_env_grammar_subset():
    # parsed in a child process because the library caches its environment
    import subprocess
    import sys
    code = (
        "import sys; sys.path.insert(0, %r); import ring_allreduce_reduce_amd as ra;"
        "print(ra.ringar_plan(1 << 30, 'float32', 8).proto, ra.ringar_plan(8, 'float32', 8).proto)" % ROOT)
    out = {}
    for v in ["LL", "^LL,LL128", "simple", "LL128"]:
        env = dict(os.environ, RINGAR_PROTO=v)
        out[v] = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                                check=True).stdout.split()
    assert out["LL"] == ["0", "0"]
    assert out["^LL,LL128"] == ["2", "2"]
    assert out["simple"] == ["2", "2"]
    assert out["LL128"] == ["1", "1"]


SLOT_DATA = {"Simple": 32768, "LL": 8192, "LL128": 30720}
SLOT_FIFO = {"Simple": lambda b: b, "LL": lambda b: 2 * b, "LL128": lambda b: -(-b // 120) * 128}


def test_parts_never_exceed_half_the_fifo():
    # a primitive's part must fit in half the FIFO depth, else the ring could
    # fill every FIFO at once and deadlock; the plan adds lanes to keep it so
    for proto, slot in SLOT_DATA.items():
        for chunk in [16, 4096, 65536, 1 << 19, 1 << 20]:
            if proto != "Simple" and chunk > (1 << 20):
                continue
            for count in [1 << 20, 1 << 26]:
                plan = ra.ringar_plan(count, "float32", 8, 16, proto, ra.make_config(chunk_bytes=chunk))
                # the largest chunk of any loop: a full chunk, or the last
                # loop's share when the channel holds less than n chunks
                per_channel = -(-count // 16) * 4
                first = chunk if per_channel >= 8 * chunk else -(-(-(-per_channel // 8)) // 16) * 16
                part = -(-first // plan.lanes)
                gran = 960 if proto == "LL128" else 1024     # lane parts: 8 whole lines under LL128
                part = -(-part // gran) * gran
                assert plan.fifo_depth in (2, 4, 8)
                assert -(-part // slot) <= plan.fifo_depth // 2, (proto, chunk, plan.lanes, plan.fifo_depth)
    # forcing too few lanes for the chunk is refused
    cfg = ra.make_config(chunk_bytes=1 << 19, lanes=1)
    with pytest.raises(ra.RingarError) as e:
        ra.ringar_plan(1 << 26, "float32", 8, 16, "Simple", cfg)
    assert e.value.code == ra.INVALID_USAGE
    # a chunk no lane count can split small enough is an invalid argument
    with pytest.raises(ra.RingarError) as e:
        ra.ringar_plan(1 << 28, "float32", 8, 1, "LL", ra.make_config(chunk_bytes=8 << 20))
    assert e.value.code == ra.INVALID_ARGUMENT


def test_fifo_depth_follows_the_footprint_budget():
    # the deepest of 8, 4, 2 slots whose in-flight footprint (wavefronts x
    # depth x FIFO bytes of one step) stays within 128 MiB (LL128: 256 MiB), unless the part
    # needs more slots
    seen = set()
    for proto in SLOT_DATA:
        for count in [1 << 12, 1 << 18, 1 << 22, 1 << 24, 1 << 26]:
            for nch in [1, 8, 16, 32]:
                for n in [2, 8]:
                    plan = ra.ringar_plan(count, "float32", n, nch, proto)
                    waves = n * plan.nchannels * plan.lanes
                    per_ch = plan.channel_elems
                    first = (plan.chunk_elems if per_ch >= n * plan.chunk_elems
                             else -(-(-(-max(1, per_ch) // n)) // 4) * 4)
                    part = -(-(first * 4) // plan.lanes)
                    gran = 960 if proto == "LL128" else 1024
                    part = -(-part // gran) * gran
                    slices = -(-part // SLOT_DATA[proto])
                    step = SLOT_FIFO[proto](min(part, SLOT_DATA[proto]))
                    d = plan.fifo_depth
                    budget = (256 if proto == "LL128" else 128) << 20    # LL128 runs fewer, longer lanes
                    seen.add(d)
                    assert slices <= d // 2
                    if d < 8:   # it was halved: the deeper FIFO was over budget
                        assert waves * 2 * d * step > budget, (proto, count, nch, n, d)
                    if d > 2:   # it was kept: within budget, or the part needs it
                        assert waves * d * step <= budget or slices > d // 4, (proto, count, nch, n, d)
    assert seen == {2, 4, 8}
    # the 64 MiB, 16-channel case: 4096 wavefronts x 16 KiB steps
    plan = ra.ringar_plan(1 << 24, "float32", 8, 16, "Simple", ra.make_config(chunk_bytes=1 << 19))
    assert (plan.lanes, plan.fifo_depth) == (32, 2)


def test_fifo_depth_knob():
    for bad in (1, 3, 16, -2):
        with pytest.raises(ra.RingarError) as e:
            ra.ringar_plan(1 << 20, "float32", 8, 4, "Simple", ra.make_config(fifo_depth=bad))
        assert e.value.code == ra.INVALID_ARGUMENT
    for d in (2, 4, 8):
        assert ra.ringar_plan(1 << 20, "float32", 8, 4, "Simple", ra.make_config(fifo_depth=d)).fifo_depth == d
    # a 64 KiB part (two slots) cannot run on a 2-slot FIFO
    cfg = ra.make_config(chunk_bytes=1 << 16, lanes=1, fifo_depth=2)
    with pytest.raises(ra.RingarError) as e:
        ra.ringar_plan(1 << 24, "float32", 8, 1, "Simple", cfg)
    assert e.value.code == ra.INVALID_USAGE
    assert ra.ringar_plan(1 << 24, "float32", 8, 1, "Simple",
                          ra.make_config(chunk_bytes=1 << 16, lanes=1, fifo_depth=4)).fifo_depth == 4


def test_small_form_rule():
    # the straight-line form serves LL and Simple when every lane part is at
    # most 1 KiB (one 16-byte packet per lane and step); the lane count rounds
    # up so that chunks of a few KiB still split into 1 KiB parts
    for proto in ("LL", "Simple", "LL128"):
        for count in [1, 100, 2048, 4096, 12345, 1 << 16, 1 << 18, 1 << 22, 1 << 24]:
            for nch in [1, 4, 16]:
                plan = ra.ringar_plan(count, "float32", 8, nch, proto)
                per_ch = plan.channel_elems
                first = (plan.chunk_elems if per_ch >= 8 * plan.chunk_elems
                         else -(-(-(-max(1, per_ch) // 8)) // 4) * 4)
                part = -(-(first * 4) // plan.lanes)
                gran = 960 if proto == "LL128" else 1024
                part = -(-part // gran) * gran
                assert plan.small_slices == int(proto != "LL128" and part <= 1024), (proto, count, nch)
                if proto != "LL128" and first * 4 <= 32 * 1024:
                    assert plan.small_slices == 1, (proto, count, nch, plan.lanes)
    cfg = ra.make_config(force_general=1)
    assert ra.ringar_plan(4096, "float32", 8, 1, "LL", cfg).small_slices == 0


def test_block_map_rule_and_grid():
    # XCD-major up to 512 KiB per rank (LL128: 32 KiB), linear above; the
    # XCD-major grid holds whole rounds of 8 groups of members (ring: the n
    # ring indices; tree: its 2n - 1 roles)
    for proto, limit in (("LL", 512 << 10), ("Simple", 512 << 10), ("LL128", 32 << 10)):
        for algo in ("ring", "tree"):
            for nbytes in (8, 4096, limit, limit + 16, 4 << 20):
                for nch in (0, 3):
                    cfg = ra.make_config(algo=algo)
                    plan = ra.ringar_plan(nbytes // 4, "float32", 8, nch, proto, cfg)
                    assert plan.xcd_major == int(nbytes <= limit), (proto, algo, nbytes, nch)
                    members = (plan.tree_waves_per_lane if plan.tree_split else 15) if algo == "tree" else 8
                    lpb = 4 if plan.lanes % 4 == 0 else 2 if plan.lanes % 2 == 0 else 1
                    groups = plan.nchannels * (plan.lanes // lpb)
                    want = 8 * members * -(-groups // 8) if plan.xcd_major else members * groups
                    assert plan.workgroups == want, (proto, algo, nbytes, nch)
    for m in (1, 2):
        plan = ra.ringar_plan(1 << 20, "float32", 8, 5, "Simple", ra.make_config(block_map=m))
        assert plan.xcd_major == (m == 2)
    for bad in (-1, 3):
        with pytest.raises(ra.RingarError) as e:
            ra.ringar_plan(1024, "float32", 8, 1, "LL", ra.make_config(block_map=bad))
        assert e.value.code == ra.INVALID_ARGUMENT


def test_xcd_major_padding_stays_resident():
    # the XCD-major grid pads the groups to whole rounds of 8; by size, a call
    # whose padded grid would exceed the 4096 resident wavefronts takes the
    # linear mapping, and a forced XCD-major mapping of it is refused
    seen_fallback = False
    for n in (2, 3, 5, 8, 10, 12, 16, 23, 33, 64):
        for nbytes in (8, 4096, 131072, 262144, 524288):
            for proto in ("auto", "LL", "Simple"):
                for algo in ("ring", "tree", "auto"):
                    cfg = ra.make_config(algo=algo)
                    try:
                        p = ra.ringar_plan(max(1, nbytes // 4), "float32", n, 0, proto, cfg)
                    except ra.RingarError:
                        continue
                    assert p.workgroups * p.threads_per_group // 64 <= 4096, (n, nbytes, proto, algo)
                    try:
                        f = ra.ringar_plan(max(1, nbytes // 4), "float32", n, 0, proto,
                                           ra.make_config(algo=algo, block_map=2))
                        assert f.xcd_major and f.workgroups * f.threads_per_group // 64 <= 4096
                    except ra.RingarError as e:
                        assert e.code == ra.INVALID_USAGE
                        assert not p.xcd_major, (n, nbytes, proto, algo)
                        seen_fallback = True
    assert seen_fallback
    # n = 10, 128 KiB: the tree's 25 channels x 2 lane blocks pad to 56 groups
    p = ra.ringar_plan(1 << 15, "float32", 10, 0, "Simple", ra.make_config(algo="tree"))
    assert (p.nchannels, p.lanes, p.xcd_major) == (25, 8, 0)
    assert p.workgroups == 19 * 50


def test_halves_buffer_rules_before_any_device_call():
    n, count = 4, 1000
    E = ra
    blk = count * 4
    # ReduceScatter: sends hold n blocks, receives one
    s = _fake(n, step=1 << 24)
    r = _fake(n, base=1 << 40, step=1 << 24)
    rs = lambda s_, r_, c=count: ra.ringar_reduce_scatter_ex(s_, r_, c, "float32", "sum", n, 2, "Simple", 0)
    assert rs(s, [0] * n) == E.INVALID_ARGUMENT
    assert rs(s, r, 0) == E.SUCCESS
    r_ip = [s[q] + q * blk for q in range(n)]            # in place: own block of own input
    assert ra.ringar_plan_coll("reduce_scatter", count, "float32", n, 2, "Simple").nchannels == 2
    r_bad = list(r_ip)
    r_bad[1] = s[1]                                      # rank 1's output on block 0 of its input
    assert rs(s, r_bad) == E.INVALID_USAGE
    r_bad = list(r)
    r_bad[2] = s[0] + 3 * blk                            # inside another rank's input
    assert rs(s, r_bad) == E.INVALID_USAGE
    r_bad = list(r)
    r_bad[3] = r[0] + 8                                  # two outputs overlap
    assert rs(s, r_bad) == E.INVALID_USAGE
    # AllGather: sends hold one block, receives n
    ag = lambda s_, r_: ra.ringar_all_gather_ex(s_, r_, count, "float32", n, 2, "Simple", 0)
    s_ip = [r[q] + q * blk for q in range(n)]            # in place: own block of own output
    s_bad = list(s_ip)
    s_bad[2] = r[2]
    assert ag(s_bad, r) == E.INVALID_USAGE
    s_bad = list(s)
    s_bad[0] = r[1] + 4 * blk - 16                       # inside another rank's output
    assert ag(s_bad, r) == E.INVALID_USAGE
    r_bad = list(r)
    r_bad[1] = r[0] + blk                                # outputs of n blocks overlap
    assert ag(s, r_bad) == E.INVALID_USAGE
    s_mis = list(s)
    s_mis[0] += 2
    assert ag(s_mis, r) == E.INVALID_ARGUMENT
    assert ra.ringar_all_gather_ex(s, r, count, "float32", 0, 2, "Simple", 0) == E.INVALID_ARGUMENT


def test_halves_plan_rule():
    # n-1 ring steps and all n blocks counted as the call's size; the channel
    # split applies to one block; AllGather plans bytes
    m = golden_model_dict()
    for coll in ("reduce_scatter", "all_gather"):
        for count in [1, 1000, 1 << 16, 1 << 20, 1 << 24]:
            for n in (2, 8):
                plan = ra.ringar_plan_coll(coll, count, "float32", n)
                total = n * count * 4
                maxc = min(m["max_channels"], m["max_pairs"] // n)
                times = [_halves_time(m, n, maxc, p, total) for p in range(3)]
                assert plan.predicted_us[:] == pytest.approx(times, rel=1e-12)
                best = min(range(3), key=lambda p: (times[p], -p))
                assert plan.proto == best, (coll, count, n)
                es = 1 if coll == "all_gather" else 4
                per = -(-(count * 4 // es) // plan.nchannels)
                per = -(-per // (16 // es)) * (16 // es)
                assert plan.channel_elems == per
                loops = max(1, -(-per // plan.chunk_elems))
                assert plan.max_steps % (loops * n) == 0
    # the AllReduce plan is unchanged by the new entry point
    a = ra.ringar_plan(1 << 20, "float32", 8)
    b = ra.ringar_plan_coll("allreduce", 1 << 20, "float32", 8)
    assert (a.proto, a.nchannels, a.lanes, a.max_steps) == (b.proto, b.nchannels, b.lanes, b.max_steps)


def _halves_time(m, n, nch, p, nbytes):
    bus = nch * m["bw_per_channel"]
    if p == 0:
        bus = min(m["ll_max_bw"], bus * m["eff"][0])
    elif p == 1:
        bus = min(bus * m["eff"][1], nch * m["ll128_per_channel_max_bw"])
    else:
        bus *= m["eff"][2]
    steps = n - 1
    return m["base_lat_us"][p] + steps * m["hw_lat_us"][p] + nbytes / (1000.0 * bus * n / steps)


def test_one_rank_ignores_fifo_knobs():
    # one rank's call is a copy: a forced lane count or FIFO depth that its
    # parts would not fit is not a reason to refuse it
    for proto in ("LL", "LL128", "Simple"):
        ra.ringar_plan(1 << 20, "int32", 1, 1, proto, ra.make_config(fifo_depth=2))
        ra.ringar_plan(1 << 20, "int32", 1, 1, proto, ra.make_config(lanes=1))
    # with two ranks the same knobs are refused
    with pytest.raises(ra.RingarError) as e:
        ra.ringar_plan(1 << 20, "int32", 2, 1, "Simple", ra.make_config(lanes=1))
    assert e.value.code == ra.INVALID_USAGE

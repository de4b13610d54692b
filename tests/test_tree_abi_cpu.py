"""Host logic of the tree AllReduce in the C-ABI library, on the CPU: the
library's tree builder equals the oracle's, its plan has the tree's geometry,
its (algorithm, protocol) choice equals the oracle model's for the same
constants, and bad requests fail before anything reaches a GPU."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import ring_allreduce_reduce_amd as ra
from libutil import golden_model_dict, lib, lib_model, oracle_model, oracle_tree_model
from oracle import select as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
E = ra


@pytest.fixture(scope="module", autouse=True)
def _lib():
    lib()


@pytest.mark.parametrize("n", list(range(1, 65)))
def test_library_tree_equals_oracle_tree(n):
    for t in (0, 1):
        for r in range(n):
            assert ra.ringar_tree(n, t, r) == oracle.dtree(n, r, t), (n, t, r)


def test_tree_query_errors():
    for args in [(0, 0, 0), (65, 0, 0), (8, 2, 0), (8, 0, 8), (8, -1, 0)]:
        with pytest.raises(ra.RingarError):
            ra.ringar_tree(*args)


def split_waves(n):
    """Wavefronts per (channel, lane) of the split form: every vertex's
    reduce role and every other vertex's broadcast role, twice for the root's
    reduce role and for either role of a vertex with two children (both
    trees have the same count)."""
    counts = []
    for t in (0, 1):
        c = 0
        for v in range(n):
            parent, c0, c1 = ra.ringar_tree(n, t, v)
            kids = (c0 >= 0) + (c1 >= 0)
            c += 2 if (parent < 0 or kids == 2) else 1
            if parent >= 0:
                c += 2 if kids == 2 else 1
        counts.append(c)
    assert counts[0] == counts[1]
    return counts[0]


@pytest.mark.parametrize("n,count,nch,proto", [(8, 1 << 24, 16, "Simple"), (8, 1 << 15, 8, "LL"),
                                               (5, 1000, 3, "LL128"), (2, 17, 1, "Simple")])
def test_tree_plan_geometry(n, count, nch, proto):
    cfg = ra.make_config(algo="tree")
    p = ra.ringar_plan(count, "float32", n, nch, proto, cfg)
    assert p.algo == 1
    assert p.nchannels == nch
    # whole workgroups of 4, 2 or 1 lanes
    lanes_per_block = 4 if p.lanes % 4 == 0 else 2 if p.lanes % 2 == 0 else 1
    assert p.threads_per_group == 64 * lanes_per_block
    groups = nch * (p.lanes // lanes_per_block)
    # 2n - 1 roles per (channel, lane), or the split form's count; the
    # XCD-major mapping of small calls pads the groups to whole rounds of 8
    members = p.tree_waves_per_lane if p.tree_split else 2 * n - 1
    if p.tree_split:
        assert members == split_waves(n)
    assert p.workgroups == members * (-(-groups // 8) * 8 if p.xcd_major else groups)
    # the tree moves one chunk of the channel per step: a lane part is at
    # most half the FIFO
    slot = {"Simple": 32768, "LL": 8192, "LL128": 30720}[proto] // 4
    part = -(-min(p.chunk_elems, p.channel_elems) // p.lanes)
    part = -(-part // 256) * 256
    assert -(-part // slot) <= p.fifo_depth // 2
    assert list(p.predicted_us) == list(p.predicted_tree_us)
    ring = ra.ringar_plan(count, "float32", n, nch, proto)
    assert ring.algo == 0 and list(ring.predicted_us) == list(ring.predicted_ring_us)


def test_tree_is_allreduce_only():
    cfg = ra.make_config(algo="tree")
    for coll in ("reduce_scatter", "all_gather"):
        with pytest.raises(ra.RingarError) as e:
            ra.ringar_plan_coll(coll, 1024, "float32", 8, 0, "auto", cfg)
        assert e.value.code == E.INVALID_ARGUMENT
    # AUTO picks the ring for the halves
    p = ra.ringar_plan_coll("reduce_scatter", 1024, "float32", 8, 0, "auto", ra.make_config(algo="auto"))
    assert p.algo == 0
    cfg = ra.make_config()
    cfg.algo = 7
    with pytest.raises(ra.RingarError):
        ra.ringar_plan(1024, "float32", 8, 0, "auto", cfg)


def _perturbed(d, k):
    """The golden model with tree constants spread out so that every
    candidate wins somewhere in a size sweep."""
    d = dict(d)
    d.update(tree_allreduce_eff=[0.92, 0.8, 1.1][k], tree_ll_divisor=[2.0, 3.8, 1.5][k],
             tree_ll128_factor=[0.94, 7 / 9, 0.5][k], tree_per_channel_max_bw=[1e9, 6.0, 9.0][k],
             tree_ll128_per_channel_max_bw=[1e9, 4.0, 2.0][k],
             tree_base_lat_us=[[3.0, 5.0, 4.0], [6.8, 14.0, 8.4], [2.0, 9.0, 3.0]][k],
             tree_hw_lat_us=[[1.0, 2.0, 1.2], [0.6, 1.25, 4.0], [3.0, 1.0, 2.0]][k],
             tree_correction=[0, 1, 1][k])
    return d


@pytest.mark.parametrize("k", [0, 1, 2])
@pytest.mark.parametrize("n", [2, 3, 8, 16])
def test_select_algo_matches_oracle_model(k, n):
    d = _perturbed(golden_model_dict(), k)
    m = lib_model(d)
    ring, tree = oracle_model(d), oracle_tree_model(d, n)
    for nch in (1, 4, 16):
        for nbytes in [0, 8, 1000, 1 << 12, 1 << 16, 1 << 20, 3 << 22, 1 << 26, 1 << 30]:
            a, p, t = ra.ringar_select_algo(nbytes, n, nch, m)
            (oa, op), ot = S.select_algo(ring, tree, n, nch, nbytes)
            assert (a, p) == (oa.lower(), op), (nch, nbytes)
            assert np.allclose(t, ot, rtol=1e-6, atol=0)


def test_auto_plan_follows_the_model():
    d = _perturbed(golden_model_dict(), 2)
    m = lib_model(d)
    seen = set()
    for nbytes in [8, 1 << 12, 1 << 16, 1 << 20, 1 << 24, 1 << 28]:
        a, p, _ = ra.ringar_select_algo(nbytes, 8, 0, m)
        plan = ra.ringar_plan(nbytes // 4, "float32", 8, 0, "auto", ra.make_config(algo="auto", model=m))
        assert (ra.ALGO_NAMES[plan.algo], ra.PROTO_NAMES[plan.proto]) == (a, p)
        seen.add(a)
        # a forced protocol keeps the faster algorithm for that protocol
        for fp in ("LL", "Simple"):
            plan = ra.ringar_plan(nbytes // 4, "float32", 8, 0, fp, ra.make_config(algo="auto", model=m))
            times = [plan.predicted_tree_us[ra.PROTOS[fp]], plan.predicted_ring_us[ra.PROTOS[fp]]]
            want = "tree" if times[0] < times[1] else "ring"
            assert ra.ALGO_NAMES[plan.algo] == want
    assert seen == {"ring", "tree"}


def test_algo_env_grammar():
    code = (
        "import sys; sys.path.insert(0, %r); import ring_allreduce_reduce_amd as ra;"
        "a = [ra.ringar_select_algo(b, 8)[0] for b in (8, 1 << 30)]; print(*a)" % ROOT)
    out = {}
    for v in ["tree", "^tree", "ring", "Tree,Ring"]:
        env = dict(os.environ, RINGAR_ALGO=v)
        out[v] = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                                check=True).stdout.split()
    assert out["tree"] == ["tree", "tree"]
    assert out["^tree"] == ["ring", "ring"]
    assert out["ring"] == ["ring", "ring"]


def test_tree_buffer_errors_before_any_device_call():
    n, count = 4, 256
    s = [0x10000 * (i + 1) for i in range(n)]
    r = [0x100000 * (i + 1) for i in range(n)]
    cfg = ra.make_config(algo="tree")
    r2 = list(r)
    r2[2] = r2[1]
    assert ra.ringar_allreduce_ex(s, r2, count, "float32", "sum", n, 2, "Simple", 0, cfg) == E.INVALID_USAGE
    r3 = list(r)
    r3[0] = 0
    assert ra.ringar_allreduce_ex(s, r3, count, "float32", "sum", n, 2, "Simple", 0, cfg) == E.INVALID_ARGUMENT
    assert ra.ringar_allreduce_ex(s, r, 0, "float32", "sum", n, 2, "Simple", 0, cfg) == E.SUCCESS


def test_default_tree_model_is_the_documented_one():
    m = ra.model_dict(ra.ringar_default_model())
    d = golden_model_dict()
    for k in ("tree_allreduce_eff", "tree_per_channel_max_bw", "tree_ll_divisor", "tree_ll128_factor",
              "tree_ll128_per_channel_max_bw", "tree_base_lat_us", "tree_hw_lat_us", "tree_correction"):
        assert m[k] == d[k], k


def test_direct_form_is_planned_only_where_it_applies():
    d = ra.make_config(direct=1)
    p = ra.ringar_plan(1 << 20, "float32", 8, 4, "Simple", d)
    assert p.direct == 1 and p.small_slices == 0
    assert ra.ringar_plan(1 << 20, "float32", 8, 4, "Simple").direct == 0
    for proto in ("LL", "LL128"):
        assert ra.ringar_plan(1 << 20, "float32", 8, 4, proto, d).direct == 0
    assert ra.ringar_plan(1 << 20, "float32", 1, 4, "Simple", d).direct == 0
    assert ra.ringar_plan(1 << 20, "float32", 8, 4, "Simple", ra.make_config(direct=1, algo="tree")).direct == 0
    assert ra.ringar_plan_coll("reduce_scatter", 1 << 17, "float32", 8, 4, "Simple", d).direct == 0
    # the small form is not used with the direct form
    small = ra.ringar_plan(64 * 8, "float32", 8, 1, "Simple", d)
    assert small.small_slices == 0 and ra.ringar_plan(64 * 8, "float32", 8, 1, "Simple").small_slices == 1
    # the library's own choice (direct = 0): only where the model picks the
    # protocol and takes Simple on the ring, from 256 KiB per rank
    for nbytes in (64 << 10, 256 << 10, 1 << 20, 64 << 20, 1 << 30):
        for algo in ("ring", "auto", "tree"):
            p = ra.ringar_plan(nbytes // 4, "float32", 8, 0, "auto", ra.make_config(algo=algo))
            want = int(p.algo == 0 and ra.PROTO_NAMES[p.proto] == "Simple" and nbytes >= 256 << 10)
            assert p.direct == want, (nbytes, algo)
    assert ra.ringar_plan(1 << 24, "float32", 8, 0, "auto").direct == 1
    assert ra.ringar_plan(1 << 24, "float32", 8, 0, "auto", ra.make_config(direct=2)).direct == 0
    assert ra.ringar_plan(1 << 24, "float32", 8, 0, "Simple").direct == 0
    assert ra.ringar_plan(1 << 24, "float32", 8, 0, "Simple", ra.make_config(direct=2)).direct == 0
    for bad in (-1, 3):
        with pytest.raises(ra.RingarError) as e:
            ra.ringar_plan(1 << 20, "float32", 8, 4, "Simple", ra.make_config(direct=bad))
        assert e.value.code == ra.INVALID_ARGUMENT


def test_tree_chunk_rule():
    # without a configured chunk the tree takes a quarter of a channel's
    # bytes, between 8 KiB (LL: 4 KiB) and 2 MiB / channels (at least 64 KiB),
    # and never above the protocol's default chunk; where the split form is
    # wanted (Simple, 256 KiB per channel or more) half a channel, up to
    # 4 MiB / channels (at least 128 KiB)
    cfg = ra.make_config(algo="tree")
    defaults = dict(zip(("LL", "LL128", "Simple"), golden_model_dict()["default_chunk_bytes"]))
    for proto in ("LL", "LL128", "Simple"):
        for nch in (1, 2, 4, 8, 16, 32):
            for mib in (0.25, 1, 4, 8, 64):
                count = int(mib * (1 << 18))
                p = ra.ringar_plan(count, "float32", 8, nch, proto, cfg)
                per = -(-count // nch)
                per = -(-per // 4) * 4
                split = proto == "Simple" and per * 4 >= 256 << 10
                hi = min(max((128 if split else 64) << 10, ((4 if split else 2) << 20) // nch), defaults[proto])
                lo = 4096 if proto == "LL" else 8192
                part = -(-(per * 4 // (2 if split else 4)) // 16) * 16
                assert p.chunk_elems * 4 == min(hi, max(lo, part)), (proto, nch, mib)
                assert p.tree_split == int(split), (proto, nch, mib)
    # a configured chunk is taken as it is
    p = ra.ringar_plan(1 << 24, "float32", 8, 16, "Simple", ra.make_config(algo="tree", chunk_bytes=512 << 10))
    assert p.chunk_elems * 4 == 512 << 10
    # the bench shape: 64 MiB per rank, 16 channels -> 256 KiB (split form)
    assert ra.ringar_plan(1 << 24, "float32", 8, 16, "Simple", cfg).chunk_elems * 4 == 256 << 10
    # a line protocol never splits and keeps the quarter rule
    assert ra.ringar_plan(1 << 24, "float32", 8, 16, "LL128", cfg).chunk_elems * 4 == 128 << 10


def test_split_form_rule():
    """The split form runs eager Simple tree calls of at least 256 KiB per
    channel; line protocols and smaller channels keep one wavefront a role."""
    cfg = ra.make_config(algo="tree")
    for nbytes, nch, want in [(8 << 20, 32, 1), (4 << 20, 32, 0), (4 << 20, 16, 1), (64 << 20, 32, 1),
                              ((8 << 20) - 4096, 32, 0)]:
        p = ra.ringar_plan(nbytes // 4, "float32", 8, nch, "Simple", cfg)
        assert p.tree_split == want, (nbytes, nch)
        assert p.tree_waves_per_lane == (split_waves(8) if want else 0)
        # every wavefront of the launch is resident at once
        assert p.lanes * p.nchannels * (p.tree_waves_per_lane or 15) <= 4096
    for proto in ("LL", "LL128"):
        p = ra.ringar_plan((64 << 20) // 4, "float32", 8, 32, proto, cfg)
        assert p.tree_split == 0 and p.tree_waves_per_lane == 0
    # the ring never splits
    p = ra.ringar_plan((64 << 20) // 4, "float32", 8, 32, "Simple", ra.make_config(algo="ring"))
    assert p.tree_split == 0


def test_split_form_env_switch():
    # RINGAR_TREE_SPLIT=0 keeps one wavefront a role (and the quarter chunk
    # rule); read in a child process because the library caches its
    # environment
    root = ROOT
    code = ("import sys; sys.path.insert(0, %r); import ring_allreduce_reduce_amd as ra;"
            "p = ra.ringar_plan(1 << 24, 'float32', 8, 32, 'Simple', ra.make_config(algo='tree'));"
            "print(p.tree_split, p.chunk_elems * 4, p.lanes)" % root)
    out = {}
    for v in ("0", "1"):
        env = dict(os.environ, RINGAR_TREE_SPLIT=v)
        out[v] = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                                check=True).stdout.split()
    assert out["0"][:2] == ["0", str(64 << 10)]
    assert out["1"][:2] == ["1", str(128 << 10)]


def test_every_automatic_plan_is_accepted():
    # no forced knob: every rank count, size, algorithm, protocol and channel
    # count has a plan (the tree's chunk cap of 2 or 4 MiB / channels is cut
    # to whole 16-byte units, which channel counts that are not powers of two
    # need: n = 9..15 at 16 MiB used to be refused)
    sizes = [8, 1024, 32768, 131072, 262144, 524288, 1 << 20, 4 << 20, 16 << 20, (64 << 20) + 48]
    for n in range(2, 65):
        for nbytes in sizes:
            for algo in ("auto", "ring", "tree"):
                for proto in ("auto", "LL", "LL128", "Simple"):
                    for nch in (0, 3, 7, 13, 32):
                        p = ra.ringar_plan(max(1, nbytes // 4), "float32", n, nch, proto, ra.make_config(algo=algo))
                        assert p.chunk_bytes % 16 == 0

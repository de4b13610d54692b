"""Pins of the oracle's double-binary-tree AllReduce (CPU only).

What ties the tree oracle to something other than itself:
  * the tree builder against the pages' figure of the two trees of 8 vertices
    (child slots included), their worked bit examples and the two-vertex case
    (tests/golden/double_tree.json);
  * the builder against an independent construction from the parent rule
    alone (tests/bruteforce_tree.py), and structural invariants for every n
    up to 64;
  * the reduction against numpy's reduction for the order-free cases, one
    IEEE operation at n = 2, the fold order written out by hand from the
    pages' figure at n = 8, a recursive brute force over the independent
    trees, the error bound, the pages' worked example, in place = out of
    place;
  * the Tree rows of the alpha-beta model against the pages' tables
    (tests/golden/tuning_tables.json).
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import select as S
from bruteforce_tree import run as brute_tree
from bruteforce_tree import tree_links
from refs import all_equal, error_bound_ok, exact_reduce, hop
from ring_allreduce_reduce_amd import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")
with open(os.path.join(GOLD, "double_tree.json")) as f:
    DT = json.load(f)
with open(os.path.join(GOLD, "tuning_tables.json")) as f:
    TT = json.load(f)["tree"]


def _links(n, t):
    return [oracle.dtree(n, r, t) for r in range(n)]


# ---------------------------------------------------------------- builder
@pytest.mark.parametrize("t", [0, 1])
def test_figure_of_eight_vertices(t):
    g = DT["n8"][f"tree{t}"]
    links = _links(8, t)
    roots = [r for r in range(8) if links[r][0] == -1]
    assert roots == [g["root"]]
    for v in range(8):
        kids = [k for k in links[v][1:] if k >= 0]
        assert kids == g["children"].get(str(v), []), f"children of {v} in tree {t}"
        for k in kids:
            assert links[k][0] == v
    internal = [v for v in range(8) if any(k >= 0 for k in links[v][1:])]
    assert sorted(internal) == sorted(g["internal"])
    assert sorted(set(range(8)) - set(internal)) == sorted(g["leaves"])


def test_bit_examples():
    for ex in DT["bit_examples_n8"]:
        u, d0, d1 = oracle.btree(8, ex["rank"])
        assert u == ex["parent"]
        assert [k for k in (d0, d1) if k >= 0] == ex["children"]
        if "child_slot" in ex:
            assert (d0, d1)[ex["child_slot"]] == ex["children"][0]


def test_two_vertices():
    for t in (0, 1):
        g = DT["n2"][f"tree{t}"]
        links = _links(2, t)
        assert [r for r in range(2) if links[r][0] == -1] == [g["root"]]
        root = g["root"]
        assert [k for k in links[root][1:] if k >= 0] == g["children"][str(root)]


def test_every_vertex_is_a_leaf_in_one_tree_at_eight():
    """The pages' point of the double tree: at 8 vertices each vertex is a
    leaf in one tree and internal in the other."""
    for v in range(8):
        leaf = [all(k < 0 for k in oracle.dtree(8, v, t)[1:]) for t in (0, 1)]
        assert leaf[0] != leaf[1]


@pytest.mark.parametrize("n", list(range(1, 65)))
def test_builder_matches_parent_rule_and_is_a_tree(n):
    for t in (0, 1):
        links = _links(n, t)
        parent, kids = tree_links(n, t)
        assert [l[0] for l in links] == parent
        assert [list(l[1:]) for l in links] == kids
        roots = [r for r in range(n) if parent[r] == -1]
        assert len(roots) == 1
        # every vertex reaches the root, within log2 steps of the bit rule
        for r in range(n):
            v, steps = r, 0
            while parent[v] != -1:
                v = parent[v]
                steps += 1
                assert steps <= max(1, n).bit_length() + 1
            assert v == roots[0]
        # parent and child links agree
        for v in range(n):
            for k in kids[v]:
                if k >= 0:
                    assert parent[k] == v
        assert sum(1 for v in range(n) for k in kids[v] if k >= 0) == n - 1


# ---------------------------------------------------------------- reduction
CASES = [(n, count, nch) for n in (2, 3, 4, 5, 7, 8) for count, nch in ((1, 1), (67, 2), (203, 3))]


@pytest.mark.parametrize("dtype", ["int8", "int32", "float16", "bfloat16", "float32", "float64"])
@pytest.mark.parametrize("op", ["sum", "prod", "min", "max"])
def test_order_free_cases_equal_numpy(dtype, op):
    if dtype in W.FLOATS and op in ("sum", "prod"):
        pytest.skip("order-dependent")
    for n, count, nch in CASES:
        xs = W.inputs(f"tree-of-{dtype}-{op}-{n}-{count}", n, count, dtype, "uniform", -4, 4)
        ys = oracle.tree_allreduce(xs, dtype, op, nch, 4 * (16 // W.ELEM_BYTES[dtype]))
        ref = exact_reduce(xs, dtype, op)
        for y in ys:
            assert np.array_equal(y.view(np.uint8), ref.view(np.uint8)), (n, count, nch)


@pytest.mark.parametrize("dtype", ["float16", "bfloat16", "float32", "float64"])
def test_two_ranks_is_one_operation(dtype):
    xs = W.inputs(f"tree-n2-{dtype}", 2, 1001, dtype, "normal")
    for nch in (1, 2, 3):
        ys = oracle.tree_allreduce(xs, dtype, "sum", nch, 16)
        ref = hop(dtype, "sum", xs[0], xs[1])
        assert all(np.array_equal(y.view(np.uint8), ref.view(np.uint8)) for y in ys)


@pytest.mark.parametrize("dtype", ["float16", "bfloat16", "float32"])
def test_fold_order_from_the_figure(dtype):
    """n = 8, two channels: channel 0 folds on tree 0, channel 1 on tree 1,
    each written out by hand from the pages' figure (own value first, then the
    children left to right)."""
    xs = W.inputs(f"tree-fig-{dtype}", 8, 1024, dtype, "normal")
    ys = oracle.tree_allreduce(xs, dtype, "sum", 2, 64)
    lo0, hi0 = oracle.channel_range(1024, dtype, 2, 0)
    lo1, hi1 = oracle.channel_range(1024, dtype, 2, 1)
    h = lambda a, b: hop(dtype, "sum", a, b)   # op(received a, local b)

    def x(r, lo, hi):
        return xs[r][lo:hi]
    # tree 0: 0 <- 4 <- {2 <- {1, 3}, 6 <- {5, 7}}
    a, b = lo0, hi0
    p2 = h(x(3, a, b), h(x(1, a, b), x(2, a, b)))
    p6 = h(x(7, a, b), h(x(5, a, b), x(6, a, b)))
    p4 = h(p6, h(p2, x(4, a, b)))
    t0 = h(p4, x(0, a, b))
    # tree 1: 7 <- 3 <- {5 <- {6, 4}, 1 <- {2, 0}}
    a, b = lo1, hi1
    p5 = h(x(4, a, b), h(x(6, a, b), x(5, a, b)))
    p1 = h(x(0, a, b), h(x(2, a, b), x(1, a, b)))
    p3 = h(p1, h(p5, x(3, a, b)))
    t1 = h(p3, x(7, a, b))
    want = np.concatenate([t0, t1])
    for y in ys:
        assert np.array_equal(y.view(np.uint8), want.view(np.uint8))


def test_three_ranks_shifted_second_tree():
    """n = 3 by hand: tree 0 is the chain 0 <- 2 <- 1; tree 1 shifts it by one
    rank: 1 <- 0 <- 2."""
    xs = W.inputs("tree-n3", 3, 512, "float32", "normal")
    ys = oracle.tree_allreduce(xs, "float32", "sum", 2, 64)
    lo1, _ = oracle.channel_range(512, "float32", 2, 1)
    x = [np.asarray(v, dtype=np.float32) for v in xs]
    want0 = (x[2][:lo1] + x[1][:lo1]) + x[0][:lo1]
    want1 = (x[0][lo1:] + x[2][lo1:]) + x[1][lo1:]
    want = np.concatenate([want0, want1])
    assert all(np.array_equal(y.view(np.uint8), want.view(np.uint8)) for y in ys)


@pytest.mark.parametrize("n", [2, 3, 4, 5, 6, 7, 8, 9, 12, 16])
def test_brute_force_recursion(n):
    rng = np.random.default_rng(n)
    for j, dtype in enumerate(["float32", "bfloat16", "float16", "float64", "int32", "int8"]):
        for op in ("sum", "prod", "min", "max"):
            count = int(rng.integers(1, 90))
            nch = int(rng.integers(1, 5))
            chunk = int(rng.integers(1, 4)) * (16 // W.ELEM_BYTES[dtype])
            dist = ("uniform", 0.9, 1.1) if (op == "prod" and dtype in W.FLOATS) else ("uniform", -4, 4)
            xs = W.inputs(f"tree-bf-{n}-{dtype}-{op}", n, count, dtype, *dist)
            got = oracle.tree_allreduce(xs, dtype, op, nch, chunk)
            want = brute_tree(xs, dtype, op, nch)
            for g, w in zip(got, want):
                assert np.array_equal(g.view(np.uint8), w.view(np.uint8)), (dtype, op, count, nch, chunk)


@pytest.mark.parametrize("dtype", ["float16", "bfloat16", "float32", "float64"])
@pytest.mark.parametrize("op", ["sum", "prod"])
def test_error_bound(dtype, op):
    n = 8
    dist = ("uniform", 0.9, 1.1) if op == "prod" else ("uniform", -4, 4)
    xs = W.inputs(f"tree-eb-{dtype}-{op}", n, 4096, dtype, *dist)
    ys = oracle.tree_allreduce(xs, dtype, op, 4, 256)
    idx = np.random.default_rng(1).choice(4096, 300, replace=False)
    assert error_bound_ok(ys[0], xs, dtype, op, idx)
    assert all_equal(ys)


def test_worked_example():
    """The pages' example (element 0 = rank, the rest 0): element 0 becomes
    n(n-1)/2 on every rank, everything else stays 0."""
    for n in (2, 4, 8):
        xs = W.inputs("worked", n, 4096, "float32", "worked")
        ys = oracle.tree_allreduce(xs, "float32", "sum", 2, 1024)
        for y in ys:
            assert y[0] == n * (n - 1) / 2 and not y[1:].any()


def test_in_place_equals_out_of_place_and_inputs_untouched():
    xs = W.inputs("tree-ip", 6, 777, "bfloat16", "normal")
    keep = [x.copy() for x in xs]
    out = oracle.tree_allreduce(xs, "bfloat16", "sum", 3, 40)
    assert all(np.array_equal(a, b) for a, b in zip(xs, keep))
    work = [x.copy() for x in xs]
    oracle.tree_allreduce(work, "bfloat16", "sum", 3, 40, out=work)
    assert all(np.array_equal(a, b) for a, b in zip(work, out))


def test_one_rank_copies():
    xs = W.inputs("tree-1", 1, 33, "float32", "normal")
    ys = oracle.tree_allreduce(xs, "float32", "sum", 1, 16)
    assert np.array_equal(ys[0], xs[0])


def test_chunk_size_changes_nothing():
    xs = W.inputs("tree-chunks", 7, 999, "float32", "normal")
    ref = oracle.tree_allreduce(xs, "float32", "sum", 2, 4)
    for chunk in (8, 12, 100, 4096):
        got = oracle.tree_allreduce(xs, "float32", "sum", 2, chunk)
        assert all(np.array_equal(a, b) for a, b in zip(got, ref))


# ---------------------------------------------------------------- model rows
def _tree_model(g, **kw):
    c = TT["constants"]
    return S.TreeModel(bw_per_channel=g["bw_per_channel"], per_channel_max_bw=g["per_channel_max_bw"],
                       ll_max_bw=g["ll_max_bw"], n_nodes=g["n_nodes"], ranks_per_node=g["ranks_per_node"],
                       base_lat=tuple(c["base_lat"]), intra_lat=tuple(c["intra_lat_nvlink"]),
                       inter_lat=tuple(c["inter_lat_net"]), **kw)


def test_a100_tree_row():
    g = TT["a100"]
    m = _tree_model(g)
    assert S.tree_bus_bw(m, g["nchannels"], "Simple") == pytest.approx(g["simple_bus_bw"], abs=0.05)
    for proto in ("LL", "LL128", "Simple"):
        assert S.tree_latency(m, proto) == pytest.approx(g["printed"][proto][0], abs=0.05)
    for proto in ("LL", "Simple"):
        assert S.tree_alg_bw(m, g["nchannels"], proto) == pytest.approx(g["printed"][proto][1], abs=0.05)
    # LL128: the page's own rule (x7/9 after the x0.92 step) gives 171.7; the
    # table prints 186.7 = 480 x 7/9 x 0.5, i.e. without the 0.92 step.
    assert S.tree_alg_bw(m, g["nchannels"], "LL128") == pytest.approx(g["ll128_alg_bw_from_code"], abs=0.05)
    assert 480 * 7 / 9 * 0.5 == pytest.approx(g["printed"]["LL128"][1], abs=0.05)


def test_machine_three_tree_rows():
    g = TT["machine_three"]
    m = _tree_model(g, tree_pattern=True)
    assert S.tree_bus_bw(m, g["nchannels"], "Simple") == pytest.approx(g["printed_simple_bus_bw"], abs=0.05)
    assert S.tree_alg_bw(m, g["nchannels"], "Simple") == pytest.approx(g["printed_simple_alg_bw"], abs=0.05)
    assert S.tree_latency(m, "Simple") == pytest.approx(g["printed_simple_lat"], abs=0.5)
    assert S.tree_latency(m, "LL") == pytest.approx(g["printed_ll_lat"], abs=0.5)
    s = S.crossover_bytes(g["printed_simple_lat"], g["printed_simple_alg_bw"],
                          g["ring_simple_lat_plateau"], g["ring_simple_alg_bw"])
    assert s / 1e6 == pytest.approx(g["printed_crossover_mb"], rel=0.01)


def test_correction_table():
    for smp in TT["correction_samples"]:
        row = S.TREE_CORRECTION[S.PROTOS.index(smp["proto"])]
        assert len(row) == 24
        assert row[smp["log_size"]] == smp["factor"]
    # applied by message size: log2(bytes / 64) = 12 is 256 KiB (LL: x0.4)
    m = S.TreeModel(bw_per_channel=20, per_channel_max_bw=24, ll_max_bw=87.7)
    plain = S.TreeModel(bw_per_channel=20, per_channel_max_bw=24, ll_max_bw=87.7, correction=False)
    nb = 64 << 12
    lat = S.tree_latency(m, "LL")
    assert (S.tree_time_us(m, 24, "LL", nb) - lat) == pytest.approx((S.tree_time_us(plain, 24, "LL", nb) - lat) / 0.4)


def test_algorithm_selection_ties_and_ids():
    ring = S.RingModel(bw_per_channel=20, ll_max_bw=87.7, ll128_per_channel_max_bw=36.7)
    tree = S.TreeModel(bw_per_channel=20, per_channel_max_bw=24, ll_max_bw=87.7)
    (algo, proto), times = S.select_algo(ring, tree, 8, 24, 1 << 30)
    assert (algo, proto) == ("Ring", "Simple") and len(times) == 6
    # small messages: the tree's LL latency (15.2) vs the ring's LL (15.0)
    (algo, proto), times = S.select_algo(ring, tree, 8, 24, 8)
    assert (algo, proto) == ("Ring", "LL")
    # an exact tie between Tree Simple and Ring Simple (n = 2, one "node",
    # equal bandwidths and latencies) goes to Ring Simple, visited first
    ring2 = S.RingModel(bw_per_channel=20, ll_max_bw=87.7, ll128_per_channel_max_bw=36.7)
    lat = S.ring_latency(ring2, 2, "Simple")
    tie = S.TreeModel(bw_per_channel=20, per_channel_max_bw=40, ll_max_bw=87.7, allreduce_eff=10.0,
                      n_nodes=1, ranks_per_node=1, base_lat=(lat, lat, lat), correction=False)
    both = (("Tree", "Simple"), ("Ring", "Simple"))
    (algo, proto), times = S.select_algo(ring2, tie, 2, 4, 1 << 20, enabled=both)
    assert times[2] == times[5] and (algo, proto) == ("Ring", "Simple")
    # only the enabled candidates compete
    (algo, proto), _ = S.select_algo(ring2, tie, 2, 4, 1 << 20, enabled=(("Tree", "Simple"),))
    assert (algo, proto) == ("Tree", "Simple")

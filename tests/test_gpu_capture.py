"""Ring AllReduce calls captured in a HIP graph and replayed, bit-exact
against the oracle on every replay: the captured form (ring and tree) numbers its steps
from zero on counters of its own and leaves every counter and flag it
consumed at zero, so each replay starts clean, while eager calls on the same
stream, made between the replays, keep their own step numbers.  Every
protocol (LL in both forms, LL128, Simple in both forms) under both
algorithms, several dtypes and ops, ragged sizes.  Each replay gets fresh inputs, copied in before it (no
clear of any library memory is recorded in the graph).  ReduceScatter and
AllGather, out of place and in place, replay bit-exact too.  The direct
form and a shape the stream has not run yet are refused under
capture, before anything is enqueued, and the capture goes on.  A graph
keeps working after eager calls on its stream have grown the FIFO memory and
counters it was captured with.  Randomly drawn calls (every knob of a ring AllReduce at
once) captured into one graph replay bit-exact too."""
import numpy as np
import pytest
import torch

import oracle
import ring_allreduce_reduce_amd as ra
from ring_allreduce_reduce_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

# (n, count, dtype, op, proto, nchannels[, algorithm])
SHAPES = [
    (8, 4096, "float32", "sum", "LL", 0),          # small LL form
    (8, 200003, "float32", "sum", "LL", 4),        # LL, ragged
    (4, 300001, "bfloat16", "sum", "LL128", 4),    # LL128, ragged
    (8, 1 << 20, "float32", "sum", "Simple", 0),   # Simple
    (3, 5000, "int32", "max", "Simple", 2),        # Simple, small form
    (5, 77777, "float16", "avg", "LL128", 3),
    (8, 4096, "float32", "sum", "LL", 0, "tree"),          # tree, small LL form
    (7, 100003, "bfloat16", "max", "LL128", 4, "tree"),
    (16, 1 << 20, "float32", "avg", "Simple", 8, "tree"),
    (5, 3000, "int8", "sum", "Simple", 2, "tree"),          # tree, small Simple form
    (6, 50001, "float64", "prod", "LL", 3, "tree"),
    (8, 1 << 20, "float32", "sum", "auto", 0),     # eager: the library's direct form; captured: FIFOs
]


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


def _cfg(shape):
    return ra.make_config(algo=shape[6]) if len(shape) > 6 else None


def _want(xs, shape):
    n, count, dtype, op, proto, nch = shape[:6]
    plan = ra.ringar_plan(count, dtype, n, nch, proto, _cfg(shape))
    run = oracle.tree_allreduce if plan.algo == 1 else oracle.ring_allreduce
    return run(xs, dtype, op, plan.nchannels, plan.chunk_elems)


def _raw(sends, recvs, shape, stream, cfg=None):
    n, count, dtype, op, proto, nch = shape[:6]
    cfg = cfg if cfg is not None else _cfg(shape)
    return ra.ringar_allreduce_ex([t.data_ptr() for t in sends], [t.data_ptr() for t in recvs], count, dtype, op,
                                  n, nch, proto, stream.cuda_stream, cfg)


def _check(recvs, want, what):
    for r, (got, w) in enumerate(zip(recvs, want)):
        assert np.array_equal(_bits(W.from_torch(got, what[2])), _bits(w)), (what, r)


def _inputs(shape, key):
    n, count, dtype, op = shape[:4]
    dist = ("uniform", 0.9, 1.1) if (op == "prod" and dtype in W.FLOATS) else ("uniform", -4, 4)
    return W.inputs(key, n, count, dtype, *dist)


def test_capture_replays_match_the_oracle():
    st = torch.cuda.Stream()
    bufs = []
    with torch.cuda.stream(st):
        for i, shape in enumerate(SHAPES):
            n, count, dtype = shape[0], shape[1], shape[2]
            xs = _inputs(shape, f"cap-warm-{i}")
            sends = [W.to_torch(x, dtype, DEV) for x in xs]
            recvs = [torch.zeros_like(s) for s in sends]
            print(f"case capture warm-up {shape}", flush=True)
            assert _raw(sends, recvs, shape, st) == ra.SUCCESS      # allocates the stream's connections
            bufs.append((sends, recvs))
    st.synchronize()
    assert ra.ringar_get_async_error(st.cuda_stream) == ra.SUCCESS
    for i, shape in enumerate(SHAPES):
        _check(bufs[i][1], _want(_inputs(shape, f"cap-warm-{i}"), shape), shape)

    g = torch.cuda.CUDAGraph()
    codes = []
    with torch.cuda.graph(g, stream=st):
        for (sends, recvs), shape in zip(bufs, SHAPES):
            codes.append(_raw(sends, recvs, shape, st))
    assert codes == [ra.SUCCESS] * len(SHAPES), [ra.ringar_result_string(c) for c in codes]

    for rep in range(4):
        xs_all = [_inputs(shape, f"cap-rep{rep}-{i}") for i, shape in enumerate(SHAPES)]
        with torch.cuda.stream(st):
            for (sends, recvs), xs, shape in zip(bufs, xs_all, SHAPES):
                for t, x in zip(sends, xs):
                    t.copy_(W.to_torch(x, shape[2], DEV))
                for t in recvs:
                    t.zero_()
        st.synchronize()
        print(f"case capture replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        assert ra.ringar_get_async_error(st.cuda_stream) == ra.SUCCESS
        for (sends, recvs), xs, shape in zip(bufs, xs_all, SHAPES):
            _check(recvs, _want(xs, shape), shape)
        # eager work on the capturing stream between replays
        shape = SHAPES[rep % len(SHAPES)]
        xs = _inputs(shape, f"cap-eager-{rep}")
        sends = [W.to_torch(x, shape[2], DEV) for x in xs]
        recvs = [torch.zeros_like(s) for s in sends]
        print(f"case capture eager between replays {shape}", flush=True)
        assert _raw(sends, recvs, shape, st) == ra.SUCCESS
        st.synchronize()
        assert ra.ringar_get_async_error(st.cuda_stream) == ra.SUCCESS
        _check(recvs, _want(xs, shape), shape)

    # back-to-back replays with no synchronisation between them: each one
    # starts from the zeros the previous one left (the inputs are those of
    # the last checked replay, so the outputs must not change)
    print("case capture 16 back-to-back replays", flush=True)
    for _ in range(16):
        g.replay()
    torch.cuda.synchronize()
    assert ra.ringar_get_async_error(st.cuda_stream) == ra.SUCCESS
    for (sends, recvs), xs, shape in zip(bufs, xs_all, SHAPES):
        _check(recvs, _want(xs, shape), shape)


def test_refused_under_capture_and_capture_goes_on():
    st = torch.cuda.Stream()
    n, count = 4, 4096
    xs = W.inputs("cap-refuse", n, count, "float32", "normal")
    sends = [W.to_torch(x, "float32", DEV) for x in xs]
    recvs = [torch.zeros_like(s) for s in sends]
    shape = (n, count, "float32", "sum", "Simple", 2)
    with torch.cuda.stream(st):
        assert _raw(sends, recvs, shape, st) == ra.SUCCESS
    st.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        refused = [
            _raw(sends, recvs, shape, st, ra.make_config(direct=1)),           # the direct form
            _raw(sends, recvs, (n, count, "float32", "sum", "LL128", 16), st),  # shape not run yet
        ]
        ok = _raw(sends, recvs, shape, st)
    assert refused == [ra.INVALID_USAGE] * 2 and ok == ra.SUCCESS
    for t in recvs:
        t.zero_()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert ra.ringar_get_async_error(st.cuda_stream) == ra.SUCCESS
    _check(recvs, _want(xs, shape), shape)


def test_replays_after_the_stream_grew_its_buffers():
    # the graph's kernels hold the FIFO and counter addresses of the capture;
    # eager calls that need more connections allocate larger buffers and keep
    # the old ones alive for the graph
    st = torch.cuda.Stream()
    small = [(4, 50000, "float32", "sum", "Simple", 2), (4, 30001, "bfloat16", "max", "LL", 2),
             (3, 40000, "int32", "sum", "LL128", 2)]
    large = [(8, 1 << 21, "float32", "sum", "Simple", 16), (8, 1 << 18, "float32", "sum", "LL", 16),
             (8, 1 << 20, "int32", "sum", "LL128", 16)]
    bufs = []
    with torch.cuda.stream(st):
        for i, shape in enumerate(small):
            sends = [W.to_torch(x, shape[2], DEV) for x in _inputs(shape, f"grow-warm-{i}")]
            recvs = [torch.zeros_like(t) for t in sends]
            print(f"case capture grow warm-up {shape}", flush=True)
            assert _raw(sends, recvs, shape, st) == ra.SUCCESS
            bufs.append((sends, recvs))
    st.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        codes = [_raw(sends, recvs, shape, st) for (sends, recvs), shape in zip(bufs, small)]
    assert codes == [ra.SUCCESS] * len(small), [ra.ringar_result_string(c) for c in codes]
    for rep, grow in enumerate(large):
        # an eager call of a larger shape on the capturing stream first
        xs = _inputs(grow, f"grow-eager-{rep}")
        sends = [W.to_torch(x, grow[2], DEV) for x in xs]
        recvs = [torch.zeros_like(t) for t in sends]
        print(f"case capture grow eager {grow}", flush=True)
        assert _raw(sends, recvs, grow, st) == ra.SUCCESS
        st.synchronize()
        assert ra.ringar_get_async_error(st.cuda_stream) == ra.SUCCESS
        _check(recvs, _want(xs, grow), grow)
        del sends, recvs
        xs_all = [_inputs(shape, f"grow-rep{rep}-{i}") for i, shape in enumerate(small)]
        with torch.cuda.stream(st):
            for (sends, recvs), xs, shape in zip(bufs, xs_all, small):
                for t, x in zip(sends, xs):
                    t.copy_(W.to_torch(x, shape[2], DEV))
                for t in recvs:
                    t.zero_()
        st.synchronize()
        print(f"case capture grow replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        assert ra.ringar_get_async_error(st.cuda_stream) == ra.SUCCESS
        for (sends, recvs), xs, shape in zip(bufs, xs_all, small):
            _check(recvs, _want(xs, shape), shape)


def _draw(rng):
    n = int(rng.integers(2, 17)) if rng.random() < 0.85 else int(rng.integers(17, 33))
    if rng.random() < 0.04:
        n = 1
    count = int(np.exp(rng.uniform(0, np.log(300_000))))
    if rng.random() < 0.04:
        count = 0
    dtype = list(W.STORAGE)[int(rng.integers(0, len(W.STORAGE)))]
    op = ["sum", "prod", "min", "max", "avg"][int(rng.integers(0, 5))]
    proto = ["LL", "LL128", "Simple", "auto"][int(rng.integers(0, 4))]
    cfg = dict(chunk_bytes=0 if rng.random() < 0.5 else int(rng.integers(1, 4096)) * 16,
               lanes=0 if rng.random() < 0.6 else int(2 ** rng.integers(0, 6)),
               fifo_depth=0 if rng.random() < 0.7 else int([2, 4, 8][rng.integers(0, 3)]),
               force_general=int(rng.random() < 0.2),
               ring_order=[int(r) for r in rng.permutation(n)] if rng.random() < 0.3 else None)
    cfg["algo"] = ["ring", "tree", "auto"][int(rng.integers(0, 3))]
    return n, count, dtype, op, proto, int(rng.integers(0, 17)), cfg, rng.random() < 0.2, rng.random() < 0.15


def _want_plan(xs, dtype, op, plan, order):
    # the tree runs over ranks 0..n-1 whatever the ring order
    if plan.algo == 1:
        return oracle.tree_allreduce(xs, dtype, op, plan.nchannels, plan.chunk_elems)
    return oracle.ring_allreduce(xs, dtype, op, plan.nchannels, plan.chunk_elems, ring=order)


def test_random_calls_captured_in_one_graph():
    rng = np.random.default_rng(606)
    st = torch.cuda.Stream()
    cases = []
    with torch.cuda.stream(st):
        for i in range(48):
            n, count, dtype, op, proto, nch, cfg, inplace, unaligned = _draw(rng)
            try:
                plan = ra.ringar_plan(count, dtype, n, nch, proto, ra.make_config(**cfg))
            except ra.RingarError:
                continue
            desc = (f"case captured random {i}: n={n} count={count} {dtype} {op} {proto} nch={nch} {cfg} "
                    f"inplace={inplace} unaligned={unaligned} -> {ra.ALGO_NAMES[plan.algo]} {ra.PROTO_NAMES[plan.proto]} "
                    f"ch={plan.nchannels} "
                    f"lanes={plan.lanes} depth={plan.fifo_depth}")
            xs = _inputs((n, count, dtype, op), f"cap-rand-warm-{i}")
            if unaligned and not inplace:
                sends = [W.to_torch(np.concatenate([np.zeros(1, x.dtype), x]), dtype, DEV)[1:] for x in xs]
                recvs = [torch.zeros(count + 1, dtype=sends[0].dtype, device=DEV)[1:] for _ in xs]
            else:
                sends = [W.to_torch(x, dtype, DEV) for x in xs]
                recvs = sends if inplace else [torch.zeros_like(t) for t in sends]
            cfgo = ra.make_config(**cfg)
            print(desc, flush=True)
            code = ra.ringar_allreduce_ex([t.data_ptr() for t in sends], [t.data_ptr() for t in recvs], count,
                                          dtype, op, n, nch, proto, st.cuda_stream, cfgo)
            if code != ra.SUCCESS:
                assert code in (ra.INVALID_ARGUMENT, ra.INVALID_USAGE), desc
                continue
            want = _want_plan(xs, dtype, op, plan, cfg["ring_order"])
            cases.append(dict(desc=desc, n=n, count=count, dtype=dtype, op=op, nch=nch, proto=proto, cfg=cfgo,
                              order=cfg["ring_order"], plan=plan, sends=sends, recvs=recvs, want=want,
                              forced_lanes=cfg["lanes"] != 0))
    st.synchronize()
    assert ra.ringar_get_async_error(st.cuda_stream) == ra.SUCCESS
    for c in cases:
        for r in range(c["n"]):
            assert np.array_equal(_bits(W.from_torch(c["recvs"][r], c["dtype"])), _bits(c["want"][r])), (c["desc"], r)
    assert len(cases) >= 36, len(cases)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        for c in cases:
            c["code"] = ra.ringar_allreduce_ex([t.data_ptr() for t in c["sends"]], [t.data_ptr() for t in c["recvs"]],
                                               c["count"], c["dtype"], c["op"], c["n"], c["nch"], c["proto"],
                                               st.cuda_stream, c["cfg"])
    # the captured line-protocol kernels hold fewer wavefronts: a plan takes
    # fewer lanes under capture, and only a forced lane count beyond that
    # residency is refused
    bad = [(c["desc"], ra.ringar_result_string(c["code"])) for c in cases
           if c["code"] != ra.SUCCESS and not (c["forced_lanes"] and c["code"] == ra.INVALID_USAGE)]
    assert not bad, bad
    cases = [c for c in cases if c["code"] == ra.SUCCESS]
    assert len(cases) >= 32, len(cases)

    for rep in range(3):
        with torch.cuda.stream(st):
            for i, c in enumerate(cases):
                xs = _inputs((c["n"], c["count"], c["dtype"], c["op"]), f"cap-rand-rep{rep}-{i}")
                for t, x in zip(c["sends"], xs):
                    t.copy_(W.to_torch(x, c["dtype"], DEV))
                if c["recvs"] is not c["sends"]:
                    for t in c["recvs"]:
                        t.zero_()
                c["want"] = _want_plan(xs, c["dtype"], c["op"], c["plan"], c["order"])
        st.synchronize()
        print(f"case captured random replay {rep} of {len(cases)} calls", flush=True)
        g.replay()
        torch.cuda.synchronize()
        assert ra.ringar_get_async_error(st.cuda_stream) == ra.SUCCESS
        for c in cases:
            for r in range(c["n"]):
                got = W.from_torch(c["recvs"][r], c["dtype"])
                assert np.array_equal(_bits(got), _bits(c["want"][r])), (rep, c["desc"], r)


# (collective, n, count per block, dtype, op, proto, nchannels, in place)
HALVES = [
    ("reduce_scatter", 8, 65536, "float32", "sum", "Simple", 4, False),
    ("reduce_scatter", 5, 30001, "bfloat16", "max", "LL", 2, False),
    ("reduce_scatter", 4, 20000, "int32", "sum", "LL128", 3, True),
    ("reduce_scatter", 3, 1000, "float64", "avg", "Simple", 0, False),   # small form
    ("all_gather", 8, 65536, "float32", None, "Simple", 4, False),
    ("all_gather", 6, 9999, "float16", None, "LL", 0, True),
    ("all_gather", 3, 50000, "int8", None, "LL128", 2, False),
]


def _halves_buffers(case, xs):
    coll, n, count, dtype, op, proto, nch, inplace = case
    sends = [W.to_torch(x, dtype, DEV) for x in xs]
    if coll == "reduce_scatter":
        recvs = ([t[r * count:(r + 1) * count] for r, t in enumerate(sends)] if inplace else
                 [torch.zeros(count, dtype=sends[0].dtype, device=DEV) for _ in range(n)])
        return sends, recvs
    full = [torch.zeros(n * count, dtype=sends[0].dtype, device=DEV) for _ in range(n)]
    if inplace:
        for r in range(n):
            full[r][r * count:(r + 1) * count].copy_(sends[r])
        sends = [full[r][r * count:(r + 1) * count] for r in range(n)]
    return sends, full


def _halves_call(case, sends, recvs, st):
    coll, n, count, dtype, op, proto, nch, inplace = case
    if coll == "reduce_scatter":
        return ra.ringar_reduce_scatter_ex([t.data_ptr() for t in sends], [t.data_ptr() for t in recvs], count,
                                           dtype, op, n, nch, proto, st.cuda_stream, None)
    return ra.ringar_all_gather_ex([t.data_ptr() for t in sends], [t.data_ptr() for t in recvs], count, dtype, n,
                                   nch, proto, st.cuda_stream, None)


def _halves_inputs(case, key):
    coll, n, count, dtype, op = case[:5]
    return W.inputs(key, n, n * count if coll == "reduce_scatter" else count, dtype, "uniform", -4, 4)


def _halves_want(case, xs):
    coll, n, count, dtype, op = case[:5]
    if coll == "reduce_scatter":
        return oracle.ring_reduce_scatter(xs, dtype, op)
    return oracle.ring_all_gather(xs, dtype)


def test_halves_captured_and_replayed():
    st = torch.cuda.Stream()
    bufs = []
    with torch.cuda.stream(st):
        for i, case in enumerate(HALVES):
            xs = _halves_inputs(case, f"cap-halves-warm-{i}")
            sends, recvs = _halves_buffers(case, xs)
            print(f"case capture halves warm-up {case}", flush=True)
            assert _halves_call(case, sends, recvs, st) == ra.SUCCESS
            bufs.append((sends, recvs, xs))
    st.synchronize()
    assert ra.ringar_get_async_error(st.cuda_stream) == ra.SUCCESS
    for (sends, recvs, xs), case in zip(bufs, HALVES):
        for got, w in zip(recvs, _halves_want(case, xs)):
            assert np.array_equal(_bits(W.from_torch(got, case[3])), _bits(w)), case
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        codes = [_halves_call(case, sends, recvs, st) for (sends, recvs, _), case in zip(bufs, HALVES)]
    assert codes == [ra.SUCCESS] * len(HALVES), [ra.ringar_result_string(c) for c in codes]
    for rep in range(3):
        xs_all = [_halves_inputs(case, f"cap-halves-rep{rep}-{i}") for i, case in enumerate(HALVES)]
        with torch.cuda.stream(st):
            for (sends, recvs, _), xs, case in zip(bufs, xs_all, HALVES):
                if not case[7]:
                    for t in recvs:
                        t.zero_()
                for t, x in zip(sends, xs):
                    t.copy_(W.to_torch(x, case[3], DEV))
        st.synchronize()
        print(f"case capture halves replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        assert ra.ringar_get_async_error(st.cuda_stream) == ra.SUCCESS
        for (sends, recvs, _), xs, case in zip(bufs, xs_all, HALVES):
            for r, (got, w) in enumerate(zip(recvs, _halves_want(case, xs))):
                assert np.array_equal(_bits(W.from_torch(got, case[3])), _bits(w)), (rep, case, r)


def test_replay_error_is_reported_after_an_eager_error_and_the_graph_recovers():
    """A replay that gives up must be reported even when an eager call on the
    stream failed, and was reported, after the capture (captured calls keep
    their capture's call id, so they record errors in a word of their own);
    reporting it clears what the failed replay left behind, so the next
    replay of a good graph is bit-exact again.  The failure is forced from
    the host: one rank's wavefronts return at once and the others give up
    after a 20 ms spin limit."""
    st = torch.cuda.Stream()
    for proto in ["Simple", "LL", "LL128"]:
        shape = (4, 100003, "float32", "sum", proto, 2)
        n, count, dtype = shape[:3]
        xs = _inputs(shape, f"cap-err-{proto}")
        sends = [W.to_torch(x, dtype, DEV) for x in xs]
        recvs = [torch.zeros_like(s) for s in sends]
        bad = ra.make_config(skip_rank=2, spin_limit_ms=20)
        print(f"case capture error {proto}: eager warm-up", flush=True)
        with torch.cuda.stream(st):
            assert _raw(sends, recvs, shape, st) == ra.SUCCESS
        st.synchronize()
        assert ra.ringar_get_async_error(st.cuda_stream) == ra.SUCCESS
        g_bad, g_good = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_bad, stream=st):
            assert _raw(sends, recvs, shape, st, bad) == ra.SUCCESS
        with torch.cuda.graph(g_good, stream=st):
            assert _raw(sends, recvs, shape, st) == ra.SUCCESS
        # an eager failure, reported, after the capture
        print(f"case capture error {proto}: eager failure", flush=True)
        with torch.cuda.stream(st):
            assert _raw(sends, recvs, shape, st, bad) == ra.SUCCESS
        st.synchronize()
        assert ra.ringar_get_async_error(st.cuda_stream) == ra.TIMEOUT
        # the failing replay is still reported
        print(f"case capture error {proto}: failing replay", flush=True)
        with torch.cuda.stream(st):
            g_bad.replay()
        st.synchronize()
        assert ra.ringar_get_async_error(st.cuda_stream) == ra.TIMEOUT
        assert ra.ringar_get_async_error(st.cuda_stream) == ra.SUCCESS
        # and a good replay afterwards starts from clean counters and flags
        for rep in range(2):
            xs2 = _inputs(shape, f"cap-err-{proto}-{rep}")
            with torch.cuda.stream(st):
                for t, x in zip(sends, xs2):
                    t.copy_(W.to_torch(x, dtype, DEV))
                for t in recvs:
                    t.zero_()
                print(f"case capture error {proto}: good replay {rep}", flush=True)
                g_good.replay()
            st.synchronize()
            assert ra.ringar_get_async_error(st.cuda_stream) == ra.SUCCESS
            _check(recvs, _want(xs2, shape), shape)
        del g_bad, g_good


@pytest.mark.parametrize("shape", [(16, 1 << 20, "float32", "avg", "Simple", 8, "tree"),
                                   (8, 1 << 21, "bfloat16", "sum", "Simple", 4, "tree")])
def test_split_tree_call_captured_after_one_eager_call(shape):
    # eagerly the tree runs these calls in its split form, whose lane count
    # differs from the captured (unsplit) form's; one eager call on a fresh
    # stream must still leave the connections the captured form needs
    n, count, dtype = shape[:3]
    plan = ra.ringar_plan(count, dtype, n, shape[5], shape[4], _cfg(shape))
    assert plan.tree_split == 1
    st = torch.cuda.Stream()
    xs = _inputs(shape, "cap-split-warm")
    sends = [W.to_torch(x, dtype, DEV) for x in xs]
    recvs = [torch.zeros_like(s) for s in sends]
    print(f"case capture split warm-up {shape}", flush=True)
    with torch.cuda.stream(st):
        assert _raw(sends, recvs, shape, st) == ra.SUCCESS
    st.synchronize()
    assert ra.ringar_get_async_error(st.cuda_stream) == ra.SUCCESS
    _check(recvs, _want(xs, shape), shape)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        code = _raw(sends, recvs, shape, st)
    assert code == ra.SUCCESS, ra.ringar_result_string(code)
    for rep in range(3):
        xs = _inputs(shape, f"cap-split-rep{rep}")
        with torch.cuda.stream(st):
            for t, x in zip(sends, xs):
                t.copy_(W.to_torch(x, dtype, DEV))
            for t in recvs:
                t.zero_()
        st.synchronize()
        print(f"case capture split replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        assert ra.ringar_get_async_error(st.cuda_stream) == ra.SUCCESS
        _check(recvs, _want(xs, shape), shape)

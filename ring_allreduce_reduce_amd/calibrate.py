"""Measures this GPU and fits the alpha-beta model of the protocol selector.

The model is the one the pages give for a ring AllReduce ([ARCH] §八.1-八.2):
a call of `bytes` per rank over n ranks and nch channels takes

    T = base + 2(n-1) * step  +  bytes / (1000 * busBw * n / (2(n-1)))   [us]

with busBw = nch * bw * eff for Simple, min(llMax, nch * bw * 0.5) for LL and
min(nch * bw * eff, nch * perChLL128) for LL128.  This tool fits, per
protocol, `base` and `step` to small calls at n = 2..8 (least squares over
2(n-1)), and the bandwidth terms to large calls at the model's largest
channel count; it keeps the pages' efficiencies and the size rule for the
channel count.  Simple's bandwidth is fitted to the direct form, which the
library runs when the model takes Simple on the ring (from 256 KiB per
rank), and the tuning table times Ring Simple that way too.  The tree AllReduce rows take the pages' Tree form with every
virtual rank one vertex ([BOOK] Japanese edition ch. 5 §四):

    T = tbase + 2 floor(log2 n) * tstep  +  bytes / (1000 * busBw * 0.5)

with busBw = nch * bw * treeEff for Simple, that / llDiv (capped at llMax)
for LL and that * ll128Factor for LL128; tbase and tstep are fitted to small
calls at n = 2..16, treeEff to 2 MiB calls, llDiv to 1 MiB calls and
ll128Factor to 8 MiB calls (where tree and ring compete).  It prints
the fitted model (the JSON layout of `ringar_model_t`) and a tuning table: for
each size the model's time per (algorithm, protocol), the measured time, and
which pair each picks.

    python -m ring_allreduce_reduce_amd.calibrate [--json out.json] [--table out.txt]
"""
from __future__ import annotations

import argparse
import json
import sys
import time

PROTOS = ("LL", "LL128", "Simple")
# smallest bytes per rank for which the library takes the direct form itself
DIRECT_AUTO_MIN_BYTES = 256 << 10


def _time_calls(ra, torch, sends, recvs, count, n, nch, proto, stream, iters, cfg=None, algo=None, direct=0):
    if algo is not None or direct:
        cfg = ra.make_config(algo=algo or "ring", direct=direct,
                             model=cfg._model_keep if cfg is not None and cfg.model else None)
    sp = [s.data_ptr() for s in sends[:n]]
    rp = [r.data_ptr() for r in recvs[:n]]

    def call():
        code = ra.ringar_allreduce_ex(sp, rp, count, "float32", "sum", n, nch, proto, stream.cuda_stream, cfg)
        if code:
            raise ra.RingarError(code, f"ringar_allreduce_ex: {ra.ringar_result_string(code)}")
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    code = ra.ringar_get_async_error(stream.cuda_stream)
    if code:
        raise ra.RingarError(code, f"asynchronous error: {ra.ringar_result_string(code)}")
    ts = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    return ts[len(ts) // 2]


def _fit_line(xs, ys):
    """Least-squares y = a + b x."""
    m = len(xs)
    sx, sy = sum(xs), sum(ys)
    sxx = sum(x * x for x in xs)
    sxy = sum(x * y for x, y in zip(xs, ys))
    b = (m * sxy - sx * sy) / (m * sxx - sx * sx)
    return (sy - b * sx) / m, b


def _flog2(x: int) -> int:
    return x.bit_length() - 1


def tree_model_time(m, n, nch, p, nbytes):
    """The model's microseconds of a tree AllReduce for protocol index p."""
    bus = min(nch * m["bw_per_channel"] * m["tree_allreduce_eff"], nch * m["tree_per_channel_max_bw"])
    if p == 0:
        bus = min(bus / m["tree_ll_divisor"], m["ll_max_bw"])
    elif p == 1:
        bus = min(bus * m["tree_ll128_factor"], nch * m["tree_ll128_per_channel_max_bw"])
    lat = m["tree_base_lat_us"][p] + 2.0 * _flog2(n) * m["tree_hw_lat_us"][p]
    return lat + nbytes / (1000.0 * bus * 0.5)


def model_time(m, n, nch, p, nbytes):
    """The model's microseconds for protocol index p (LL 0, LL128 1, Simple 2)."""
    bus = nch * m["bw_per_channel"]
    if p == 0:
        bus = min(m["ll_max_bw"], bus * m["eff"][0])
    elif p == 1:
        bus = min(bus * m["eff"][1], nch * m["ll128_per_channel_max_bw"])
    else:
        bus = bus * m["eff"][2]
    steps = 2.0 * (n - 1)
    alg = bus * n / steps
    return m["base_lat_us"][p] + steps * m["hw_lat_us"][p] + nbytes / (1000.0 * alg)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--json", help="write the fitted model here")
    ap.add_argument("--table", help="write the tuning table here")
    ap.add_argument("--nranks", type=int, default=8)
    args = ap.parse_args(argv)

    import torch
    import ring_allreduce_reduce_amd as ra

    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()
    n = args.nranks
    big = 256 << 20
    sends = [torch.randn(big // 4, device=dev) for _ in range(n)]
    recvs = [torch.empty_like(s) for s in sends]
    m = ra.model_dict(ra.ringar_default_model())
    maxc = min(m["max_channels"], m["max_pairs"] // n)
    log = lambda s: print(s, file=sys.stderr, flush=True)

    # latency: smallest calls whose chunks all hold one packet, one channel
    for p, proto in enumerate(PROTOS):
        xs, ys = [], []
        for nr in range(2, n + 1):
            us = _time_calls(ra, torch, sends, recvs, 64 * nr, nr, 1, proto, stream, 200)
            xs.append(2.0 * (nr - 1))
            ys.append(us)
        base, step = _fit_line(xs, ys)
        m["base_lat_us"][p] = round(base, 2)
        m["hw_lat_us"][p] = round(step, 3)
        log(f"{proto}: base {base:.2f} us, step {step:.3f} us")

    # bandwidth: the largest call at the largest channel count (Simple in
    # the direct form, as the library runs it when the model takes Simple)
    def bus_at(proto, p, nbytes):
        us = _time_calls(ra, torch, sends, recvs, nbytes // 4, n, maxc, proto, stream, 10,
                         direct=int(proto == "Simple"))
        lat = m["base_lat_us"][p] + 2.0 * (n - 1) * m["hw_lat_us"][p]
        alg = nbytes / (1000.0 * max(us - lat, 1e-3))
        return alg * 2.0 * (n - 1) / n
    simple = bus_at("Simple", 2, big)
    m["bw_per_channel"] = round(simple / (maxc * m["eff"][2]), 3)
    ll = bus_at("LL", 0, 64 << 20)
    m["ll_max_bw"] = round(ll, 2)
    ll128 = bus_at("LL128", 1, big)
    m["ll128_per_channel_max_bw"] = round(ll128 / maxc, 3)
    log(f"bus bandwidth at {maxc} channels: Simple {simple:.1f}, LL {ll:.1f}, LL128 {ll128:.1f} GB/s")

    # tree latency: one packet per lane, one channel, n = 2..16 (floor(log2 n) levels)
    small = [torch.randn(64 * 16, device=dev) for _ in range(16)]
    small_out = [torch.empty_like(t) for t in small]
    for p, proto in enumerate(PROTOS):
        xs, ys = [], []
        for nr in range(2, 17):
            us = _time_calls(ra, torch, small, small_out, 64 * nr, nr, 1, proto, stream, 200, algo="tree")
            xs.append(2.0 * _flog2(nr))
            ys.append(us)
        base, step = _fit_line(xs, ys)
        m["tree_base_lat_us"][p] = round(base, 2)
        m["tree_hw_lat_us"][p] = round(step, 3)
        log(f"tree {proto}: base {base:.2f} us, step per level {step:.3f} us")

    # tree bandwidth at the largest channel count, fitted at the sizes where
    # the model has to choose between tree and ring (Simple at 2 MiB per
    # rank, LL at 1 MiB, LL128 against Simple at 8 MiB): far above them the
    # ring wins anyway, and the tree runs closer to its model there than at
    # medium sizes (the pages' reason for a size correction of the tree's
    # bandwidth)
    def tree_bus_at(proto, p, nbytes):
        us = _time_calls(ra, torch, sends, recvs, nbytes // 4, n, maxc, proto, stream, 10, algo="tree")
        lat = m["tree_base_lat_us"][p] + 2.0 * _flog2(n) * m["tree_hw_lat_us"][p]
        return 2.0 * nbytes / (1000.0 * max(us - lat, 1e-3))
    tsimple = tree_bus_at("Simple", 2, 2 << 20)
    m["tree_allreduce_eff"] = round(tsimple / (maxc * m["bw_per_channel"]), 4)
    m["tree_per_channel_max_bw"] = 1e9
    tll = tree_bus_at("LL", 0, 1 << 20)
    m["tree_ll_divisor"] = round(tsimple / tll, 4) if tll < m["ll_max_bw"] else 1.0
    tll128 = tree_bus_at("LL128", 1, 8 << 20)
    m["tree_ll128_factor"] = round(tll128 / tree_bus_at("Simple", 2, 8 << 20), 4)
    m["tree_ll128_per_channel_max_bw"] = 1e9
    m["tree_correction"] = 0
    log(f"tree bus bandwidth at {maxc} channels: Simple {tsimple:.1f}, LL {tll:.1f}, LL128 {tll128:.1f} GB/s")

    # tuning table: model vs measurement, each protocol at its own channel count
    ra_model = ra.model_from_dict(m)
    cfg = ra.make_config(model=ra_model)
    rows = []
    pairs = [("Tree", q) for q in PROTOS] + [("Ring", q) for q in PROTOS]
    for sh in range(3, 29, 2):
        nbytes = 1 << sh
        count = max(1, nbytes // 4)
        line = {"bytes": nbytes}
        for a, proto in pairs:
            p = PROTOS.index(proto)
            # Ring Simple from 256 KiB per rank: the direct form, which the
            # library runs when the model picks it
            direct = int((a, proto) == ("Ring", "Simple") and nbytes >= DIRECT_AUTO_MIN_BYTES)
            pcfg = ra.make_config(model=ra_model, algo=a.lower(), direct=direct)
            plan = ra.ringar_plan(count, "float32", n, 0, proto, pcfg)
            pred = plan.predicted_us[p]
            us = _time_calls(ra, torch, sends, recvs, count, n, 0, proto, stream,
                             20 if nbytes >= (16 << 20) else 100, pcfg)
            line[(a, proto)] = (plan.nchannels, pred, us)
        # the model's pick: reverse id order, strictly smaller wins (ties to Ring Simple)
        best = None
        for pair in reversed(pairs):
            if best is None or line[pair][1] < line[best][1]:
                best = pair
        line["model_pick"] = best
        line["measured_pick"] = min(pairs, key=lambda q: line[q][2])
        rows.append(line)
        log(f"{nbytes:>10d} B: " + "  ".join(f"{a[0]}{q} {line[(a, q)][2]:.1f}/{line[(a, q)][1]:.1f}"
                                            for a, q in pairs))

    out = [f"# ring and tree AllReduce tuning table, n = {n}, fp32 sum, one MI355X ({time.strftime('%Y-%m-%d')})",
           "# command: python -m ring_allreduce_reduce_amd.calibrate --json <model.json> --table <this file>",
           "# per (algorithm, protocol): channels chosen by the size rule, model us, measured us (median,",
           "# HIP events); Ring Simple from 256 KiB per rank runs the direct form, as the library does when",
           "# the model picks it",
           "# fitted model: " + json.dumps(m), ""]
    name = lambda pr: f"{pr[0]} {pr[1]}"
    hdr = f"{'bytes/rank':>11s} | " + " | ".join(f"{name(pr):>12s} ch model  meas." for pr in pairs) + \
        " |     model pick |   fastest"
    out.append(hdr)
    for r in rows:
        cells = " | ".join(f"{r[pr][0]:>15d} {r[pr][1]:6.1f} {r[pr][2]:6.1f}" for pr in pairs)
        out.append(f"{r['bytes']:>11d} | {cells} | {name(r['model_pick']):>14s} | {name(r['measured_pick'])}")
    agree = sum(r["model_pick"] == r["measured_pick"] for r in rows)
    out.append("")
    out.append(f"model pick = fastest measured at {agree} of {len(rows)} sizes")
    text = "\n".join(out) + "\n"
    print(text)
    if args.table:
        open(args.table, "w").write(text)
    if args.json:
        with open(args.json, "w") as f:
            json.dump(m, f, indent=2)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""The protocol selector's choices against kernel time, from a rocprofv3 trace.

The tuning table of `calibrate` times each (algorithm, protocol) pair with
HIP events around each call.  This tool evidences the same choices with the
kernels' own durations as rocprofv3 records them: `run` makes, for every size
of the table (8 B to 128 MiB per rank, n = 8 or --nranks, fp32 sum) and every pair, a few
warm-up calls and then K timed calls with the built-in model's channel count
(Ring Simple from 256 KiB per rank in the direct form, which the library runs
when the model takes Simple on the ring), and writes the list of calls it
made; `summarize` reads the kernel trace of that run, assigns the library's
collective dispatches to the calls in order, and prints per size and pair the
median kernel time and the achieved memory GB/s (algorithmic bytes per call,
S (2n + 4(n-1) e) for the FIFO forms, e = 1, 2, 128/120 for Simple, LL,
LL128, and S (5n - 4) for the direct form, over the kernel time), the
model's pick and the pair the kernels ran fastest.

    cd /tmp && export TMPDIR=/tmp PYTHONPATH=<repo> && \\
        rocprofv3 --kernel-trace --output-format csv -d <dir> -o run -- \\
        python3 -m ring_allreduce_reduce_amd.tuning_trace run --calls <calls.json>
    python3 -m ring_allreduce_reduce_amd.tuning_trace summarize --trace <dir>/run_kernel_trace.csv \\
        --calls <calls.json> [--out <table.txt>]
"""
from __future__ import annotations

import argparse
import csv
import json
import statistics
import sys

PROTOS = ("LL", "LL128", "Simple")
PAIRS = [("Tree", q) for q in PROTOS] + [("Ring", q) for q in PROTOS]
SIZES = [1 << sh for sh in range(3, 29, 2)]       # 8 B .. 128 MiB per rank
DIRECT_AUTO_MIN_BYTES = 256 << 10                # the library's own direct choice
WARMUP, TIMED = 3, 20


def alg_bytes(nbytes: int, n: int, proto: str, direct: bool) -> float:
    if direct:
        return float(nbytes) * (5 * n - 4)
    e = {"Simple": 1.0, "LL": 2.0, "LL128": 128.0 / 120.0}[proto]
    return float(nbytes) * (2 * n + 4 * (n - 1) * e)


def run(calls_path: str, n: int = 8) -> int:
    import torch
    import ring_allreduce_reduce_amd as ra
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()
    biggest = max(SIZES) // 4
    sends = [torch.randn(biggest, device=dev) for _ in range(n)]
    recvs = [torch.empty_like(s) for s in sends]
    sp = [s.data_ptr() for s in sends]
    rp = [r.data_ptr() for r in recvs]
    calls = []
    for nbytes in SIZES:
        count = max(1, nbytes // 4)
        for algo, proto in PAIRS:
            direct = int((algo, proto) == ("Ring", "Simple") and nbytes >= DIRECT_AUTO_MIN_BYTES)
            cfg = ra.make_config(algo=algo.lower(), direct=direct)
            plan = ra.ringar_plan(count, "float32", n, 0, proto, cfg)
            auto = ra.ringar_plan(count, "float32", n, 0, "auto", ra.make_config(algo="auto"))
            for _ in range(WARMUP + TIMED):
                code = ra.ringar_allreduce_ex(sp, rp, count, "float32", "sum", n, 0, proto, stream.cuda_stream, cfg)
                if code:
                    raise ra.RingarError(code, "ringar_allreduce_ex")
            torch.cuda.synchronize()
            code = ra.ringar_get_async_error(stream.cuda_stream)
            if code:
                raise ra.RingarError(code, "asynchronous error")
            calls.append({"bytes": nbytes, "algo": algo, "proto": proto, "direct": direct,
                          "nchannels": plan.nchannels, "lanes": plan.lanes, "workgroups": plan.workgroups,
                          "model_us": plan.predicted_us[PROTOS.index(proto)],
                          "pick": [ra.ALGO_NAMES[auto.algo].capitalize(), ra.PROTO_NAMES[auto.proto]],
                          "dispatches": WARMUP + TIMED})
        print(f"{nbytes} B done", flush=True)
    with open(calls_path, "w") as f:
        json.dump({"n": n, "warmup": WARMUP, "timed": TIMED, "calls": calls}, f, indent=1)
    return 0


def _collective(name: str) -> bool:
    return "ringar::ring_kernel" in name or "ringar::tree_kernel" in name


def summarize(trace_path: str, calls_path: str, out_path: str | None) -> int:
    spec = json.load(open(calls_path))
    calls, n = spec["calls"], spec["n"]
    rows = [r for r in csv.DictReader(open(trace_path)) if _collective(r["Kernel_Name"])]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    want = sum(c["dispatches"] for c in calls)
    if len(rows) != want:
        print(f"trace holds {len(rows)} collective dispatches, the run made {want}", file=sys.stderr)
        return 1
    i = 0
    for c in calls:
        group = rows[i:i + c["dispatches"]]
        i += c["dispatches"]
        durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in group[spec["warmup"]:]]
        grids = {int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]) for r in group}
        if grids != {c["workgroups"]}:
            print(f"dispatch order does not match the calls at {c}", file=sys.stderr)
            return 1
        c["kernel_us"] = statistics.median(durs)
        c["gbs"] = alg_bytes(c["bytes"], n, c["proto"], bool(c["direct"])) / (c["kernel_us"] * 1e3)
    out = [f"# the selector's choices against kernel time: n = {n}, fp32 sum, one MI355X; per (algorithm, protocol)",
           "# the model's channel count, the median rocprofv3 kernel duration of 20 calls (after 3 warm-up",
           "# calls) and the achieved memory GB/s (algorithmic bytes over kernel time; '/d' = the direct form,",
           "# S (5n - 4) bytes); the model's pick (algorithm = auto, protocol = auto) and the fastest kernels",
           "# commands (from the repository root on the MI355X box):",
           "#   cd /tmp && export TMPDIR=/tmp PYTHONPATH=<repo> && \\",
           "#     rocprofv3 --kernel-trace --output-format csv -d <dir> -o run -- \\",
           f"#     python3 -m ring_allreduce_reduce_amd.tuning_trace run --calls <calls.json>" +
           ("" if n == 8 else f" --nranks {n}"),
           "#   python3 -m ring_allreduce_reduce_amd.tuning_trace summarize --trace <dir>/run_kernel_trace.csv \\",
           "#     --calls <calls.json> --out <this file>",
           ""]
    hdr = f"{'bytes/rank':>11s} | " + " | ".join(f"{a + ' ' + q:>12s} ch     us   GB/s" for a, q in PAIRS) + \
        " |     model pick |  fastest kernels"
    out.append(hdr)
    agree = 0
    for nbytes in SIZES:
        line = [c for c in calls if c["bytes"] == nbytes]
        cells = []
        for c in line:
            mark = "/d" if c["direct"] else "  "
            cells.append(f"{c['nchannels']:>13d}{mark} {c['kernel_us']:6.1f} {c['gbs']:6.0f}")
        fastest = min(line, key=lambda c: c["kernel_us"])
        pick = tuple(line[0]["pick"])
        ok = (fastest["algo"], fastest["proto"]) == pick
        agree += ok
        out.append(f"{nbytes:>11d} | " + " | ".join(cells) +
                   f" | {pick[0] + ' ' + pick[1]:>14s} | {fastest['algo'] + ' ' + fastest['proto']:>16s}")
    out += ["", f"model pick = fastest kernels at {agree} of {len(SIZES)} sizes"]
    text = "\n".join(out) + "\n"
    print(text)
    if out_path:
        open(out_path, "w").write(text)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--calls", required=True, help="write the list of calls made here (JSON)")
    r.add_argument("--nranks", type=int, default=8)
    s = sub.add_parser("summarize")
    s.add_argument("--trace", required=True, help="rocprofv3 run_kernel_trace.csv of the run")
    s.add_argument("--calls", required=True)
    s.add_argument("--out")
    args = ap.parse_args(argv)
    if args.cmd == "run":
        return run(args.calls, args.nranks)
    return summarize(args.trace, args.calls, args.out)


if __name__ == "__main__":
    sys.exit(main())

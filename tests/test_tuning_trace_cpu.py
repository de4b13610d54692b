"""The kernel-trace evidence tool's assignment of dispatches to calls (CPU,
on a synthetic trace): every collective dispatch goes to its call in order,
warm-up calls are dropped, other kernels are ignored, and a trace whose
dispatch count or grid sizes do not match the calls is refused."""
import csv
import json

from ring_allreduce_reduce_amd import tuning_trace as TT

FIELDS = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X", "Grid_Size_X"]


def _write(tmp_path, calls, durs, extra=True, grid_off=0):
    rows, t = [], 1000
    for c, d in zip(calls, durs):
        name = "void ringar::tree_kernel<x>(y)" if c["algo"] == "Tree" else "void ringar::ring_kernel<x>(y)"
        for k in range(c["dispatches"]):
            if extra:
                rows.append(["KERNEL_DISPATCH", "ringar::fill_u64_kernel(unsigned long*)", t, t + 5, 256, 256])
                t += 10
            us = 1000.0 if k < TT.WARMUP else d      # warm-up calls are slow and must be dropped
            rows.append(["KERNEL_DISPATCH", name, t, t + int(us * 1000), 64, 64 * (c["workgroups"] + grid_off)])
            t += int(us * 1000) + 100
    rows.reverse()                                   # the tool sorts by start time itself
    trace = tmp_path / "trace.csv"
    with open(trace, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(FIELDS)
        w.writerows(rows)
    return str(trace)


def _calls(tmp_path):
    calls = []
    for nbytes in TT.SIZES:
        for algo, proto in TT.PAIRS:
            calls.append({"bytes": nbytes, "algo": algo, "proto": proto, "direct": 0, "nchannels": 4,
                          "lanes": 1, "workgroups": 8 + len(calls) % 3, "model_us": 1.0,
                          "pick": ["Tree", "LL"] if nbytes < 4096 else ["Ring", "Simple"],
                          "dispatches": TT.WARMUP + TT.TIMED})
    path = tmp_path / "calls.json"
    path.write_text(json.dumps({"n": 8, "warmup": TT.WARMUP, "timed": TT.TIMED, "calls": calls}))
    return calls, str(path)


def test_dispatches_assigned_in_order(tmp_path):
    calls, cpath = _calls(tmp_path)
    # Tree LL fastest below 4 KiB, Ring Simple from there: the pick agrees at every size
    durs = [(1.0 if (c["bytes"] < 4096 and (c["algo"], c["proto"]) == ("Tree", "LL")) or
             (c["bytes"] >= 4096 and (c["algo"], c["proto"]) == ("Ring", "Simple")) else 5.0 + i % 7)
            for i, c in enumerate(calls)]
    out = tmp_path / "table.txt"
    assert TT.summarize(_write(tmp_path, calls, durs), cpath, str(out)) == 0
    text = out.read_text()
    assert f"model pick = fastest kernels at {len(TT.SIZES)} of {len(TT.SIZES)} sizes" in text
    # the achieved GB/s of the 8 MiB Ring Simple row: S (2n + 4(n-1)) bytes in 1 us
    row = [ln for ln in text.splitlines() if ln.strip().startswith(str(8 << 20))][0]
    assert f"{TT.alg_bytes(8 << 20, 8, 'Simple', False) / 1e3:6.0f}" in row


def test_mismatched_traces_are_refused(tmp_path):
    calls, cpath = _calls(tmp_path)
    durs = [2.0] * len(calls)
    # one dispatch missing
    trace = _write(tmp_path, calls, durs)
    lines = open(trace).read().splitlines()
    drop = max(i for i, ln in enumerate(lines) if "tree_kernel" in ln or "ring_kernel" in ln)
    open(trace, "w").write("\n".join(lines[:drop] + lines[drop + 1:]) + "\n")
    assert TT.summarize(trace, cpath, None) == 1
    # grid sizes that are not the calls' own
    assert TT.summarize(_write(tmp_path, calls, durs, grid_off=1), cpath, None) == 1

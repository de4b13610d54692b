"""Benchmark of the ring AllReduce hot path on one MI355X.

Workload: n = 8 virtual ranks, fp32 sum, 16M elements (64 MiB) per rank drawn
N(0, 1), Simple protocol, 16 channels, 512 KiB chunks, ring r -> r+1 mod 8.
One step = one ring AllReduce over all 8 ranks with inputs resident in HBM.

Prints one JSON line: busbw (value), algbw, the dominant kernel's roofline
(algorithmic bytes per launch / average launch time measured with HIP events
on the launch stream, against MI355X's 8 TB/s HBM peak), and beside it the
memory system's measured ceilings: a plain device copy moving the same bytes
(its buffers far exceed the 256 MB Infinity Cache, so it streams from HBM),
a copy whose buffers stay in the Infinity Cache, and the rate of the bytes no
schedule can avoid (each rank reads its input and writes its output once).
The CPU baseline is the oracle timed on this host, single-threaded and with
its channels spread over host threads (the host's CPU model and core count
are reported); the oracle's output also checks the last timed call bit for
bit.

Other workloads of the same kind: `--dtype`, `--proto`, `--nchannels`
(0 = the size rule), `--chunk-bytes` (0 = the protocol default) and
`--bytes-per-rank` (e.g. the bf16 LL128 workload at 64 MiB:
`--dtype bfloat16 --proto LL128 --nchannels 0 --chunk-bytes 0`).
`--coll reduce_scatter` / `--coll all_gather` time the two halves of the
ring on the same shape instead (8 ranks, 64 MiB n-block buffer per rank, 8 MiB
blocks); their busbw is algbw x (n-1)/n.  `--algo tree` times the tree
AllReduce (double binary tree, channel c on tree c % 2) on the AllReduce
workload; its busbw keeps the AllReduce convention algbw x 2(n-1)/n.
`--direct` times the direct form of the ring AllReduce (Simple, each slice
written straight into the successor's receive buffer, no FIFO).
`--sweep` prints a table instead of the JSON line: every workload's sizes
(int32 Simple at 4 ranks; the LL sweep at 8 channels; the bf16 LL128 sweep
with automatic channels; the automatic protocol over 8 B .. 1 GiB per rank,
ring only and with the model choosing ring or tree), each timed with HIP
events (median) and reported as busbw and algorithmic memory GB/s (a
protocol marked "/d" ran the direct form, which the library takes for calls
whose protocol the model picks, and its bytes are the direct form's).
"""
import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "busbw & achieved HBM GB/s (% of peak), fp32 sum, n=8 virtual ranks, 64 MiB"
HBM_PEAK_GBS = 8000.0
NRANKS = 8
BYTES_PER_RANK = 64 << 20
NCHANNELS = 16
CHUNK_BYTES = 512 * 1024
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ring_simple_fp32_64MiB_n8_traffic.txt")
# counter summaries of the other 64 MiB AllReduce forms, by (algorithm, direct, protocol, dtype)
TRAFFIC_FILES = {
    ("ring", False, "Simple", "float32"): TRAFFIC_FILE,
    ("ring", True, "Simple", "float32"): os.path.join(ROOT, "profiles", "ring_direct_fp32_64MiB_n8_traffic.txt"),
    ("ring", False, "LL128", "bfloat16"): os.path.join(ROOT, "profiles", "ring_ll128_bf16_64MiB_n8_traffic.txt"),
    ("tree", False, "Simple", "float32"): os.path.join(ROOT, "profiles", "tree_simple_fp32_64MiB_n8_traffic.txt"),
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash():
    """Hash of the device code: the kernel sources (`.hip` files and the
    headers they include) with comments and whitespace removed, so that a
    comment edit or a host-side change leaves a counter record valid."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "ring_allreduce_reduce_amd", "csrc")
    for p in sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.h"))):
        with open(p) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(os.path.basename(p).encode())
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def plan_key(cfg):
    """The launch shape a counter record was taken with."""
    return f"lanes={cfg['lanes']} fifo_depth={cfg['fifo_depth']} workgroups={cfg['workgroups']}"


def read_traffic(cfg, path=TRAFFIC_FILE):
    """Measured HBM bytes per launch from a committed counter summary, if it
    was taken on the current kernel code with the same launch shape."""
    if path is None or not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_hash:\s*(\w+)", text)
    m_plan = re.search(r"plan:\s*([^\n]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or not m_plan or m_hash.group(1) != kernel_source_hash():
        return None
    if m_plan.group(1).strip() != plan_key(cfg):
        return None
    return float(m_bytes.group(1))


def alg_bytes(n, s, e=1.0, coll="allreduce"):
    """Algorithmic bytes of one ring call over n ranks.  AllReduce of s bytes
    per rank: every rank reads its send buffer once and writes its receive
    buffer once, and each of the 2(n-1) steps writes and reads one chunk
    through a FIFO whose bytes are e times the payload (Simple 1, LL 2, LL128
    128/120).  The tree AllReduce moves the same bytes: each of the n-1
    non-root vertices sends the whole buffer up once and receives it down
    once through a FIFO, 4(n-1) e s in all, plus the 2n s of user buffers.  ReduceScatter / AllGather with s bytes in the n-block buffer of
    each rank: every rank reads its input once (s, resp. s/n), writes its
    output once (s/n, resp. s), and each of the n-1 steps writes and reads one
    block through the FIFO."""
    if coll == "allreduce":
        return s * (2 * n + 4 * (n - 1) * e)
    if coll == "direct":
        # per ring index and chunk C: send 2C, n-2 x recvReduceSend 3C,
        # recvReduceCopySend 4C, n-2 x recvCopySend 2C, recv 0 (the data is
        # already in place): C (5n - 4); over the n ring indices s (5n - 4)
        return s * (5 * n - 4)
    return n * s + s + 2 * (n - 1) * s * e


FIFO_EXPANSION = {"LL": 2.0, "LL128": 128.0 / 120.0, "Simple": 1.0}


def sweep(reps_small=200, reps_big=20):
    """One table line per (workload, size); see the module docstring."""
    import torch

    import ring_allreduce_reduce_amd as ra

    dev = torch.device("cuda:0")
    st = torch.cuda.Stream()
    tdt = {"int32": torch.int32, "float32": torch.float32, "bfloat16": torch.bfloat16}

    def timed(n, count, dtype, proto, nch, chunk=0, algo="ring"):
        if dtype == "int32":
            xs = [torch.randint(-1000, 1001, (count,), dtype=torch.int32, device=dev) for _ in range(n)]
        else:
            xs = [torch.randn(count, device=dev).to(tdt[dtype]) for _ in range(n)]
        ys = [torch.empty_like(x) for x in xs]
        cfg = ra.make_config(chunk_bytes=chunk, algo=algo)
        sp, rp = [x.data_ptr() for x in xs], [y.data_ptr() for y in ys]
        plan = ra.ringar_plan(count, dtype, n, nch, proto, cfg)

        def call():
            code = ra.ringar_allreduce_ex(sp, rp, count, dtype, "sum", n, nch, proto, st.cuda_stream, cfg)
            if code:
                raise RuntimeError(ra.ringar_result_string(code))
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        es = xs[0].element_size()
        reps = reps_big if count * es >= (8 << 20) else reps_small
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(st)
            call()
            b.record(st)
        torch.cuda.synchronize()
        if ra.ringar_get_async_error(st.cuda_stream):
            raise RuntimeError("asynchronous error")
        t = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)[reps // 2]
        del xs, ys
        s = count * es
        pname = ra.PROTO_NAMES[plan.proto]
        alg = s / (t * 1e-6) / 1e9
        # the direct form (the library's choice for calls whose protocol the
        # model picks) moves S (5n - 4) bytes instead of the FIFO form's
        b_alg = alg_bytes(n, s, coll="direct") if plan.direct else alg_bytes(n, s, FIFO_EXPANSION[pname])
        hbm = b_alg / (t * 1e-6) / 1e9
        return dict(bytes=s, us=t, proto=pname + ("/d" if plan.direct else ""), algo=ra.ALGO_NAMES[plan.algo],
                    nch=plan.nchannels, algbw=alg, busbw=alg * 2 * (n - 1) / n, hbm=hbm)

    rows = []

    def emit(name, r):
        line = (f"{name:34s} {r['bytes']:>11d} {r['algo']:>5s} {r['proto']:>8s} {r['nch']:>4d} "
                f"{r['us']:>10.1f} {r['algbw']:>8.2f} {r['busbw']:>8.2f} {r['hbm']:>8.1f} "
                f"{100 * r['hbm'] / HBM_PEAK_GBS:>6.1f}")
        rows.append(line)
        print(line, flush=True)

    print(f"{'workload':34s} {'bytes/rank':>11s} {'algo':>5s} {'proto':>8s} {'nch':>4s} {'us':>10s} "
          f"{'algbw':>8s} {'busbw':>8s} {'hbmGB/s':>8s} {'%peak':>6s}", flush=True)
    emit("int32 sum n=4 Simple 2ch 16KiB", timed(4, 65536, "int32", "Simple", 2, 16384))
    emit("fp32 sum n=8 Simple 16ch 512KiB", timed(8, 16 << 20, "float32", "Simple", 16, 512 << 10))
    for sh in range(13, 21):
        emit("fp32 sum n=8 LL 8ch", timed(8, (1 << sh) // 4, "float32", "LL", 8))
    for sh in range(20, 27):
        emit("bf16 sum n=8 LL128 auto ch", timed(8, (1 << sh) // 2, "bfloat16", "LL128", 0))
    for sh in range(3, 31, 3):
        emit("fp32 sum n=8 auto (ring)", timed(8, max(1, (1 << sh) // 4), "float32", "auto", 0))
    for sh in range(3, 31, 3):
        emit("fp32 sum n=8 auto (ring or tree)", timed(8, max(1, (1 << sh) // 4), "float32", "auto", 0,
                                                     algo="auto"))
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (for scaling memory counters)")
    ap.add_argument("--coll", default="allreduce", choices=["allreduce", "reduce_scatter", "all_gather"],
                    help="the AllReduce (default) or one of its halves on the same 8 x 64 MiB shape")
    ap.add_argument("--algo", default="ring", choices=["ring", "tree"],
                    help="AllReduce algorithm: the ring (default) or the double binary tree")
    ap.add_argument("--sweep", action="store_true",
                    help="print a table over every workload's sizes instead of the JSON line")
    ap.add_argument("--direct", action="store_true",
                    help="the ring AllReduce's direct form (no FIFO: the successor's receive buffer)")
    ap.add_argument("--dtype", default="float32", choices=["int8", "int32", "float16", "bfloat16", "float32",
                                                           "float64"],
                    help="element type of the AllReduce (default fp32, the headline workload)")
    ap.add_argument("--proto", default="Simple", choices=["Simple", "LL", "LL128", "auto"])
    ap.add_argument("--nchannels", type=int, default=NCHANNELS, help="0 = the model's size rule")
    ap.add_argument("--chunk-bytes", type=int, default=CHUNK_BYTES, help="0 = the protocol's default")
    ap.add_argument("--bytes-per-rank", type=int, default=BYTES_PER_RANK)
    ap.add_argument("--cpu-threads", type=int, default=16,
                    help="most host threads for the channel-parallel oracle timing")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the {NRANKS} ranks are virtual ranks inside one MI355X; "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    if args.sweep:
        sweep()
        return

    import numpy as np
    import torch

    import ring_allreduce_reduce_amd as ra
    oracle = None
    if not args.no_cpu_baseline:
        import oracle
    from ring_allreduce_reduce_amd import workloads as W

    coll = args.coll
    algo = args.algo if coll == "allreduce" else "ring"
    direct = bool(args.direct) and coll == "allreduce" and algo == "ring"
    dtype, proto, nch = args.dtype, args.proto, args.nchannels
    if coll == "all_gather" or coll == "reduce_scatter":
        dtype = "float32"
    es = W.ELEM_BYTES[dtype]
    s = args.bytes_per_rank
    count = s // es                           # elements in the (n-block) buffer of a rank
    block = count // NRANKS
    headline = (coll == "allreduce" and algo == "ring" and not direct and dtype == "float32" and
                proto == "Simple" and nch == NCHANNELS and args.chunk_bytes == CHUNK_BYTES and
                s == BYTES_PER_RANK)
    log("generating inputs")
    dev = torch.device("cuda:0")
    # the headline workload keeps its own seed key; others draw by shape
    key = "config2" if dtype == "float32" and s == BYTES_PER_RANK else f"bench-{dtype}-{s}"
    if coll == "all_gather":
        xs = W.inputs(key + "-ag", NRANKS, block, dtype, "normal")
        sends = [W.to_torch(x, dtype, dev) for x in xs]
        recvs = [torch.empty(count, device=dev) for _ in sends]
    else:
        xs = W.inputs(key, NRANKS, count, dtype, "normal")
        sends = [W.to_torch(x, dtype, dev) for x in xs]
        recvs = [torch.empty_like(t) if coll == "allreduce" else torch.empty(block, device=dev) for t in sends]
    stream = torch.cuda.Stream()
    # the tree moves a whole chunk per channel up and then down: it takes its
    # own chunk rule rather than the ring's 512 KiB
    chunk_cfg = 0 if algo == "tree" and args.chunk_bytes == CHUNK_BYTES else args.chunk_bytes
    cfg = ra.make_config(chunk_bytes=chunk_cfg, algo=algo, direct=int(direct))
    plan = ra.ringar_plan_coll(coll, count if coll == "allreduce" else block, dtype, NRANKS, nch, proto, cfg)
    pname = ra.PROTO_NAMES[plan.proto]
    chunk_bytes = plan.chunk_bytes
    send_ptrs = [t.data_ptr() for t in sends]
    recv_ptrs = [t.data_ptr() for t in recvs]

    def step():
        if coll == "allreduce":
            code = ra.ringar_allreduce_ex(send_ptrs, recv_ptrs, count, dtype, "sum", NRANKS, nch,
                                          proto, stream.cuda_stream, cfg)
        elif coll == "reduce_scatter":
            code = ra.ringar_reduce_scatter_ex(send_ptrs, recv_ptrs, block, dtype, "sum", NRANKS,
                                               nch, proto, stream.cuda_stream, cfg)
        else:
            code = ra.ringar_all_gather_ex(send_ptrs, recv_ptrs, block, dtype, NRANKS, nch,
                                           proto, stream.cuda_stream, cfg)
        if code != 0:
            raise RuntimeError(f"{coll}: {ra.ringar_result_string(code)}")

    torch.cuda.synchronize()
    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if ra.ringar_get_async_error(stream.cuda_stream) != 0:
        raise RuntimeError("warmup call reported an error")

    log(f"timing {args.steps} steps")
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_all0.record(stream)
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    t_all1.record(stream)
    torch.cuda.synchronize()
    code = ra.ringar_get_async_error(stream.cuda_stream)
    if code != 0:
        raise RuntimeError(f"timed calls reported {ra.ringar_result_string(code)}")
    total_ms = t_all0.elapsed_time(t_all1)
    per_launch_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    ms_per_step = total_ms / args.steps
    avg_launch_ms = sum(per_launch_ms) / len(per_launch_ms)
    log(f"ms/step {ms_per_step:.4f}  avg launch {avg_launch_ms:.4f} ms  min {min(per_launch_ms):.4f}")

    e = FIFO_EXPANSION[pname]
    b_alg = alg_bytes(NRANKS, s, e, coll="direct" if direct else coll)
    achieved = b_alg / (avg_launch_ms * 1e-3) / 1e9
    # the bytes no schedule can avoid: every rank reads its input and writes
    # its output once (2 n S for the AllReduce)
    b_user = (2 * NRANKS * s) if coll == "allreduce" else (NRANKS * s + s)
    user_gbs = b_user / (avg_launch_ms * 1e-3) / 1e9

    # Plain device copies on the same stream, for the memory system's
    # practical ceilings: (a) a copy moving the kernel's algorithmic bytes
    # (read B/2 + write B/2; far larger than the 256 MB Infinity Cache, so it
    # streams from HBM), (b) a copy whose two buffers total 128 MiB (the ring
    # FIFO footprint; it stays in the Infinity Cache between repetitions).
    def copy_rate(nbytes, reps):
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            for _ in range(3):
                dst.copy_(src)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(reps)]
            for a, b in ev:
                a.record(stream)
                dst.copy_(src)
                b.record(stream)
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
        del src, dst
        torch.cuda.empty_cache()
        return 2 * nbytes / (t * 1e-3) / 1e9, t

    if args.copy_calibration:
        # three plain 256 MiB copies of known size, to scale memory counters
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
        log("copy calibration: 3 x 256 MiB device copies")
    copy_hbm_gbs, copy_hbm_ms = copy_rate(int(b_alg // 2) // 4096 * 4096, 10)
    copy_cache_gbs, _ = copy_rate(64 << 20, 50)
    log(f"device copy: {copy_hbm_gbs:.0f} GB/s at {int(b_alg // 2) >> 20} MiB, "
        f"{copy_cache_gbs:.0f} GB/s at 64 MiB (in cache)")

    algbw = s / (ms_per_step * 1e-3) / 1e9
    bus_factor = (2 if coll == "allreduce" else 1) * (NRANKS - 1) / NRANKS
    busbw = algbw * bus_factor
    tfile = TRAFFIC_FILES.get((algo, bool(direct), pname, dtype)) \
        if coll == "allreduce" and s == BYTES_PER_RANK else None
    traffic = read_traffic({"lanes": plan.lanes, "fifo_depth": plan.fifo_depth,
                            "workgroups": plan.workgroups}, tfile)

    def run_oracle(threaded=False, threads=1):
        if coll == "allreduce" and algo == "tree":
            return oracle.tree_allreduce(xs, dtype, "sum", plan.nchannels, plan.chunk_elems), 1
        if coll == "allreduce":
            if threaded:
                return oracle.ring_allreduce_threaded(xs, dtype, "sum", plan.nchannels, plan.chunk_elems,
                                                      threads=threads)
            return oracle.ring_allreduce(xs, dtype, "sum", plan.nchannels, plan.chunk_elems), 1
        if coll == "reduce_scatter":
            return oracle.ring_reduce_scatter(xs, dtype, "sum"), 1
        return oracle.ring_all_gather(xs, dtype), 1

    def host_cpu():
        model = "unknown"
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
        avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
        return {"model": model, "logical_cpus": os.cpu_count(), "available_to_process": avail}

    def time_oracle(seconds, threaded, threads):
        t0 = time.perf_counter()
        want, used = run_oracle(threaded, threads)
        calls = 1
        while time.perf_counter() - t0 < seconds and calls < 500:
            run_oracle(threaded, threads)
            calls += 1
        return want, used, (time.perf_counter() - t0) / calls, calls

    cpu = None
    if not args.no_cpu_baseline:
        oracle.load()
        hc = host_cpu()
        log(f"host CPU: {hc['model']}, {hc['available_to_process']} of {hc['logical_cpus']} logical CPUs "
            f"available; timing the CPU oracle (single thread, then channels over threads)")
        want, _, dt1, calls1 = time_oracle(10.0, False, 1)
        threads = max(1, min(args.cpu_threads, hc["available_to_process"] or 1))
        want_t, used, dtn, callsn = time_oracle(10.0, True, threads)
        got = [W.from_torch(r, dtype) for r in recvs]
        same = all(np.array_equal(g.view(np.uint8), w.view(np.uint8)) for g, w in zip(got, want))
        same_t = all(np.array_equal(a.view(np.uint8), b.view(np.uint8)) for a, b in zip(want, want_t))
        if not same:
            raise RuntimeError("GPU result differs from the CPU oracle")
        if not same_t:
            raise RuntimeError("the channel-threaded oracle differs from the single-threaded one")
        log(f"oracle {dt1:.3f} s per call (1 thread, {calls1} calls), {dtn:.3f} s ({used} threads, "
            f"{callsn} calls); GPU output matches bit for bit")
        cpu = {"value": round(s / dtn / 1e9 * bus_factor, 4), "unit": "GB/s", "cores": used,
               "kind": "oracle", "seconds_per_call": round(dtn, 4), "calls": callsn,
               "sample": f"the full workload ({NRANKS} ranks x {s >> 20} MiB {dtype}) repeated {callsn} times "
                         f"(~10 s), the C oracle with its channels spread over {used} threads; value is busbw",
               "single_thread": {"value": round(s / dt1 / 1e9 * bus_factor, 4), "cores": 1,
                                 "seconds_per_call": round(dt1, 4), "calls": calls1},
               "host_cpu": hc}

    what = {"allreduce": (f"{algo} AllReduce" + (" (direct form)" if direct else ""), f"{s >> 20} MiB per rank"),
            "reduce_scatter": ("ring ReduceScatter", f"{s >> 20} MiB input per rank ({NRANKS} blocks)"),
            "all_gather": ("ring AllGather", f"{(s // NRANKS) >> 20} MiB input, {s >> 20} MiB output per rank")}[coll]
    dname = {"int8": "int8", "int32": "int32", "float16": "fp16", "bfloat16": "bf16", "float32": "fp32",
             "float64": "fp64"}[dtype]
    metric = METRIC if headline else \
        f"busbw & achieved memory GB/s (% of 8 TB/s), {what[0]}, {dname} sum, n={NRANKS} virtual ranks, " \
        f"{s >> 20} MiB, {pname}"
    out = {
        "metric": metric,
        "value": round(busbw, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"int8": "i8", "int32": "i32", "float16": "f16", "bfloat16": "bf16", "float32": "f32",
                  "float64": "f64"}[dtype],
        "data": "synthetic",
        "config": {"workload": f"{what[0]}, {NRANKS} virtual ranks, {dname}"
                               f"{' sum' if coll != 'all_gather' else ''}, {what[1]}, {pname}, "
                               f"{plan.nchannels} channels, {chunk_bytes >> 10} KiB chunks",
                   "nranks": NRANKS, "bytes_per_rank": s, "proto": pname, "nchannels": plan.nchannels,
                   "chunk_bytes": chunk_bytes, "lanes": plan.lanes, "fifo_depth": plan.fifo_depth,
                   "workgroups": plan.workgroups},
        "algbw_gbs": round(algbw, 3),
        "busbw_gbs": round(busbw, 3),
        "hbm_alg_gbs": round(achieved, 1),
        "hbm_frac_of_peak": round(achieved / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "memory", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "bound_detail": "HBM3E plus the 256 MB Infinity Cache: the user buffers stream from HBM, "
                                     "the FIFO traffic stays largely in the Infinity Cache; the L2-side counters "
                                     "behind traffic cannot tell the two apart",
                     "alg_bytes_per_launch": b_alg, "avg_launch_ms": round(avg_launch_ms, 5),
                     "user_buffer_bytes_per_launch": b_user, "user_buffer_gbs": round(user_gbs, 1),
                     "copy_gbs": round(copy_hbm_gbs, 1), "frac_of_copy": round(achieved / copy_hbm_gbs, 4),
                     "copy_bytes": int(b_alg // 2) // 4096 * 4096 * 2,
                     "copy_in_cache_gbs": round(copy_cache_gbs, 1)},
        "cpu_baseline": cpu,
        # The figures the pages give for NVIDIA systems ([ARCH] introduction),
        # quoted beside the measurement as model constants: none was measured here.
        "pages_model_constants": {"source": "[ARCH] introduction", "kind": "model constants, not measurements",
                                  "nvlink_bidirectional_gbs_per_gpu": {"A100": 600, "H100": 900},
                                  "protocol_payload_efficiency": {"Simple": 1.0, "LL128": 0.94, "LL": 0.5}},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

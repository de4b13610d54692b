"""Alpha-beta protocol model of the ring and tree AllReduce: test
infrastructure only.

A plain transcription of the tuning model on the pages, restricted to the Ring
and Tree algorithms and their three protocols:

  [ARCH] arganzheng.life, "NCCL architecture: topology, channels, algorithms
         and protocols": §八.1 (ncclTopoTuneModel: per-protocol bus bandwidth,
         latency = base + steps x per-step hardware latency, algorithm
         bandwidth = bus bandwidth x n / (2(n-1)) for AllReduce), §八.2
         (ncclTopoGetAlgoTime: time = latency + bytes / (1000 x bandwidth),
         the fastest enabled candidate wins), §六.4 (shrinking the channel
         count while bytes < channels x threads x per-thread threshold).
  [BOOK] aireadcode.com, "NCCL Source Code Deep Dive" (Japanese edition,
         ch. 5 §一): candidates are pushed to the front of a list in id order
         and the first strictly smaller time wins, so on a tie the candidate
         enumerated last wins: Simple, then LL128, then LL.

  [BOOK] Japanese edition, ch. 5 §四 (tree.cc): the Tree rows only serve
         AllReduce; bus bandwidth = min(channels x bw x 0.92, channels x
         per-channel tree cap), LL divided by 3.8 and capped at the LL
         maximum, LL128 times 7/9 on one node (120/128 across nodes) and
         capped per channel; latency = base + 2 x ((ranks per node - 1) x
         intra-node step + log2(nodes) x inter-node step); the Tree
         correction table scales the bandwidth by message size; [ARCH] §八.1
         adds the x0.85 of the TREE pattern and the algorithm bandwidth =
         bus bandwidth x 0.5.  The candidate ids run Tree LL, Tree LL128,
         Tree Simple, Ring LL, Ring LL128, Ring Simple (the model map), so on
         a tie Ring Simple wins first and Tree LL last.

Protocol order everywhere is the pages' protocol table order: LL, LL128,
Simple.  Bandwidths are GB/s, times microseconds, sizes bytes.
"""
from __future__ import annotations

from dataclasses import dataclass, field

PROTOS = ("LL", "LL128", "Simple")


@dataclass
class RingModel:
    """Inputs of the Ring rows of the tuning model (one node, one ring)."""
    bw_per_channel: float                  # per-channel bandwidth found for the ring graph
    ll_max_bw: float                       # absolute cap on LL bus bandwidth
    ll128_per_channel_max_bw: float        # per-channel cap on LL128 bus bandwidth
    eff: tuple = (0.5, 0.92, 1.0)          # payload efficiency per protocol
    base_lat: tuple = (6.6, 14.0, 8.4)     # per-call latency per protocol
    hw_lat: tuple = (0.6, 1.9, 3.4)        # per-ring-step latency per protocol
    max_channels: int = 32                 # channel count before the size rule
    max_pairs: int = 256                   # cap on nranks x channels (co-residency)
    threads: tuple = (512, 640, 512)       # threads per channel per protocol
    thread_threshold: tuple = (8, 8, 64)   # bytes per thread (LL: times nranks on a ring)
    default_chunk_bytes: tuple = (32768, 491520, 524288)
    extra: dict = field(default_factory=dict)


def ring_bus_bw(m: RingModel, nchannels: int, proto: str) -> float:
    """Bus bandwidth of the ring under `proto` ([ARCH] §八.1)."""
    p = PROTOS.index(proto)
    bus = nchannels * m.bw_per_channel
    if proto == "LL":
        return min(m.ll_max_bw, bus * m.eff[p])
    if proto == "LL128":
        return min(bus * m.eff[p], nchannels * m.ll128_per_channel_max_bw)
    return bus * m.eff[p]


def ring_alg_bw(m: RingModel, nranks: int, nchannels: int, proto: str) -> float:
    """Algorithm bandwidth: bus bandwidth x nranks / nsteps, nsteps = 2(n-1)."""
    nsteps = 2 * (nranks - 1)
    return ring_bus_bw(m, nchannels, proto) * nranks / nsteps


def ring_latency(m: RingModel, nranks: int, proto: str) -> float:
    """Latency: base + nsteps x per-step hardware latency (one node)."""
    p = PROTOS.index(proto)
    return m.base_lat[p] + 2 * (nranks - 1) * m.hw_lat[p]


def ring_time_us(m: RingModel, nranks: int, nchannels: int, proto: str, nbytes: int) -> float:
    """Predicted time of one AllReduce of nbytes per rank ([ARCH] §八.2)."""
    bw = ring_alg_bw(m, nranks, nchannels, proto)
    return ring_latency(m, nranks, proto) + nbytes / (1000.0 * bw)


def select(m: RingModel, nranks: int, nchannels: int, nbytes: int, enabled=PROTOS):
    """Fastest enabled protocol and the three predicted times.

    Candidates are visited in reverse enumeration order (the list is built by
    pushing to the front) and replaced only on a strictly smaller time.
    """
    times = [ring_time_us(m, nranks, nchannels, p, nbytes) for p in PROTOS]
    best, best_t = None, float("inf")
    for p in reversed(PROTOS):
        if p not in enabled:
            continue
        t = times[PROTOS.index(p)]
        if t < best_t:
            best, best_t = p, t
    if best is None:
        raise ValueError("no protocol enabled")
    return best, times


def max_channels(m: RingModel, nranks: int) -> int:
    return max(1, min(m.max_channels, m.max_pairs // max(1, nranks)))


def auto_channels(m: RingModel, nranks: int, proto: str, nbytes: int, start: int | None = None) -> int:
    """Shrink the channel count while each thread would get too few bytes
    ([ARCH] §六.4).  The count never drops below one."""
    p = PROTOS.index(proto)
    nc = start if start is not None else max_channels(m, nranks)
    thr = m.thread_threshold[p] * (nranks if proto == "LL" else 1)
    while nc > 1 and nbytes < nc * m.threads[p] * thr:
        nc -= 1
    return nc


def resolve(m: RingModel, nranks: int, nbytes: int, nchannels: int = 0,
            proto: str | None = None, chunk_bytes: int = 0):
    """Resolve an AUTO call: protocol (model argmin over the channel count the
    model sees), then the channel count (size rule), then the chunk size (the
    protocol's default).  Returns (proto, nchannels, chunk_bytes)."""
    if nranks == 1:
        return "Simple", 1, chunk_bytes or m.default_chunk_bytes[2]
    model_nch = nchannels if nchannels > 0 else max_channels(m, nranks)
    if proto is None:
        proto, _ = select(m, nranks, model_nch, nbytes)
    if nchannels <= 0:
        nchannels = auto_channels(m, nranks, proto, nbytes)
    if chunk_bytes <= 0:
        chunk_bytes = m.default_chunk_bytes[PROTOS.index(proto)]
    return proto, nchannels, chunk_bytes


def crossover_bytes(lat1: float, bw1: float, lat2: float, bw2: float) -> float:
    """Message size where lat1 + S/(1000 bw1) == lat2 + S/(1000 bw2)."""
    return 1000.0 * (lat2 - lat1) / (1.0 / bw1 - 1.0 / bw2)


# ---------------------------------------------------------------- Tree rows
ALGOS = ("Tree", "Ring")

# Bandwidth correction of the Tree AllReduce by message size, per protocol
# (LL, LL128, Simple), indexed by log2(bytes / 64) ([BOOK] Japanese edition,
# ch. 5 §四, cost_model.cc table; the pages' measured "tree efficiency curve").
TREE_CORRECTION = (
    (1.0, 1.0, 1.0, 1.0, .9, .8, .7, .7, .7, .7, .6, .5, .4, .4, .5, .6, .7, .8, .9, 1.0, 1.0, 1.0, 1.0, 1.0),
    (1.0, 1.0, 1.0, 1.0, 1.0, .9, .8, .8, .8, .7, .6, .6, .6, .6, .6, .6, .8, .9, .9, .9, .9, 1.0, 1.0, 1.0),
    (.9, .9, .9, .9, .9, .9, .9, .8, .7, .6, .6, .5, .5, .5, .5, .6, .7, .8, .7, .7, .8, .9, .9, .9),
)


@dataclass
class TreeModel:
    """Inputs of the Tree rows of the tuning model."""
    bw_per_channel: float                  # per-channel bandwidth of the tree graph
    per_channel_max_bw: float              # perChMaxTreeBw
    ll_max_bw: float                       # absolute cap on LL bus bandwidth
    per_channel_max_ll128_bw: float = 1e30 # perChMaxTreeLL128Bw (no cap when unknown)
    allreduce_eff: float = 0.92
    ll_divisor: float = 3.8
    n_nodes: int = 1
    ranks_per_node: int = 8
    tree_pattern: bool = False             # the TREE pattern's extra x0.85
    base_lat: tuple = (6.8, 14.0, 8.4)     # per-call latency per protocol
    intra_lat: tuple = (0.6, 1.25, 4.0)    # per step inside a node (NVLink table)
    inter_lat: tuple = (5.0, 8.5, 14.0)    # per step between nodes (network table)
    correction: bool = True                # apply TREE_CORRECTION
    ll128_factor: float | None = None      # None: the pages' 7/9 (one node) or 120/128


def log2i(x: int) -> int:
    """Floor of log2 for x >= 1; -1 for x < 1."""
    return x.bit_length() - 1 if x >= 1 else -1


def tree_bus_bw(m: TreeModel, nchannels: int, proto: str) -> float:
    """Bus bandwidth of the Tree AllReduce under `proto`."""
    bus = nchannels * m.bw_per_channel
    bus = min(bus * m.allreduce_eff, nchannels * m.per_channel_max_bw)
    if proto == "LL":
        bus = min(bus / m.ll_divisor, m.ll_max_bw)
    elif proto == "LL128":
        f = m.ll128_factor if m.ll128_factor is not None else (7.0 / 9.0 if m.n_nodes == 1 else 120.0 / 128.0)
        bus = min(bus * f, nchannels * m.per_channel_max_ll128_bw)
    if m.tree_pattern:
        bus *= 0.85
    return bus


def tree_alg_bw(m: TreeModel, nchannels: int, proto: str) -> float:
    """Algorithm bandwidth of the Tree AllReduce: bus bandwidth x 0.5."""
    return tree_bus_bw(m, nchannels, proto) * 0.5


def tree_latency(m: TreeModel, proto: str) -> float:
    """base + 2 x ((ranks per node - 1) x intra step + log2(nodes) x inter step)."""
    p = PROTOS.index(proto)
    return m.base_lat[p] + 2 * ((m.ranks_per_node - 1) * m.intra_lat[p] + log2i(m.n_nodes) * m.inter_lat[p])


def tree_time_us(m: TreeModel, nchannels: int, proto: str, nbytes: int) -> float:
    """Predicted time of one Tree AllReduce of nbytes per rank, with the size
    correction of the bandwidth when enabled."""
    bw = tree_alg_bw(m, nchannels, proto)
    ls = log2i(nbytes >> 6)
    if m.correction and 0 <= ls < 23:
        bw *= TREE_CORRECTION[PROTOS.index(proto)][ls]
    return tree_latency(m, proto) + nbytes / (1000.0 * bw)


def select_algo(ring: RingModel, tree: TreeModel, nranks: int, nchannels: int, nbytes: int,
                enabled=(("Tree", "LL"), ("Tree", "LL128"), ("Tree", "Simple"),
                         ("Ring", "LL"), ("Ring", "LL128"), ("Ring", "Simple"))):
    """Fastest enabled (algorithm, protocol) and the six predicted times in
    id order (Tree LL, LL128, Simple, Ring LL, LL128, Simple).  Candidates are
    visited in reverse id order and replaced only on a strictly smaller
    time."""
    times = [tree_time_us(tree, nchannels, p, nbytes) for p in PROTOS] + \
            [ring_time_us(ring, nranks, nchannels, p, nbytes) for p in PROTOS]
    ids = [(a, p) for a in ALGOS for p in PROTOS]
    best, best_t = None, float("inf")
    for i in reversed(range(len(ids))):
        if ids[i] not in enabled:
            continue
        if times[i] < best_t:
            best, best_t = ids[i], times[i]
    if best is None:
        raise ValueError("no algorithm/protocol enabled")
    return best, times

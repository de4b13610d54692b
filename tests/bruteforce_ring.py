"""Brute-force ring AllReduce: one thread per ring index, real bounded FIFOs.

Written from the pages' description of the protocol rather than from the
oracle: every ring index runs the runRing primitive sequence (send,
recvReduceSend x (n-2), recvReduceCopySend, recvCopySend x (n-2), recv) over a
FIFO of NCCL_STEPS = 8 slots to its successor.  Messages carry their chunk id
and a step flag; a receiver checks that flags arrive as step + 1, in order,
and takes the chunk it works on from the message, not from a formula.  The
only scheduling rule a rank knows is its first send: its own chunk (i-1).

Pure Python: for tiny inputs only.
"""
from __future__ import annotations

import queue
import threading

import numpy as np

from refs import hop
from ring_allreduce_reduce_amd.workloads import ELEM_BYTES

NCCL_STEPS = 8


def _loops(count: int, esize: int, n: int, nch: int, chunk: int):
    """(channel, [chunk (start, end) for k in 0..n-1]) for every loop, walking
    each channel's contiguous range from its start."""
    unit = 16 // esize
    per = -(-count // nch)
    per = -(-per // unit) * unit
    for c in range(nch):
        start = min(count, c * per)
        end = min(count, start + per)
        pos = start
        while pos < end:
            left = end - pos
            if left >= n * chunk:
                size = chunk
            else:
                size = -(-(-(-left // n)) // unit) * unit
            spans = []
            for k in range(n):
                a = min(end, pos + k * size)
                b = min(end, pos + (k + 1) * size)
                spans.append((a, b))
            yield c, spans
            pos += min(left, n * chunk)


def run(xs, dtype: str, op: str, nchannels: int, chunk_elems: int, ring=None):
    n = len(xs)
    count = xs[0].size
    ring = list(range(n)) if ring is None else list(ring)
    ys = [np.zeros_like(x) for x in xs]
    if n == 1:
        ys[0][:] = xs[0]
        return ys
    loops = list(_loops(count, ELEM_BYTES[dtype], n, nchannels, chunk_elems))
    fifo = [queue.Queue(maxsize=NCCL_STEPS) for _ in range(n)]   # fifo[i]: into ring index i
    errors = []

    def rank(i: int):
        me = ring[i]
        x, y = xs[me], ys[me]
        out_q, in_q = fifo[(i + 1) % n], fifo[i]
        sent = [0]
        recvd = [0]

        def send(k, v):
            sent[0] += 1
            out_q.put((sent[0], k, v.copy()), timeout=30)

        def recv():
            flag, k, v = in_q.get(timeout=30)
            recvd[0] += 1
            if flag != recvd[0]:
                raise RuntimeError(f"ring index {i}: flag {flag} != step {recvd[0]}")
            return k, v

        try:
            for _, spans in loops:
                def own(k):
                    a, b = spans[k]
                    return x[a:b]

                def put(k, v):
                    a, b = spans[k]
                    y[a:b] = v

                k = (i - 1) % n
                send(k, own(k))
                for _ in range(n - 2):
                    k, v = recv()
                    send(k, hop(dtype, op, v, own(k)))
                k, v = recv()
                fin = hop(dtype, op, v, own(k))
                put(k, fin)
                send(k, fin)
                for _ in range(n - 2):
                    k, v = recv()
                    put(k, v)
                    send(k, v)
                k, v = recv()
                put(k, v)
        except Exception as exc:  # noqa: BLE001 - reported by the caller
            errors.append(exc)

    threads = [threading.Thread(target=rank, args=(i,)) for i in range(n)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    if errors:
        raise errors[0]
    return ys

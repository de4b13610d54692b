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

from refs import divide, hop, hop_op
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
                    send(k, hop(dtype, hop_op(op), v, own(k)))
                k, v = recv()
                fin = hop(dtype, hop_op(op), v, own(k))
                if op == "avg":
                    fin = divide(dtype, fin, n)
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


def _block_loops(count: int, esize: int, nch: int, chunk: int):
    """Pieces [a, b) of a block of `count` elements, one per (channel, loop):
    the block splits over channels like a buffer, and each loop takes up to
    `chunk` elements of every block at once."""
    unit = 16 // esize
    per = -(-count // nch)
    per = -(-per // unit) * unit
    for c in range(nch):
        start = min(count, c * per)
        end = min(count, start + per)
        pos = start
        while pos < end:
            b = min(end, pos + chunk)
            yield pos, b
            pos = b


def _threads(n, body):
    fifo = [queue.Queue(maxsize=NCCL_STEPS) for _ in range(n)]   # fifo[i]: into ring index i
    errors = []

    def rank(i):
        out_q, in_q = fifo[(i + 1) % n], fifo[i]
        st = {"sent": 0, "recvd": 0}

        def send(k, v):
            st["sent"] += 1
            out_q.put((st["sent"], k, v.copy()), timeout=30)

        def recv():
            flag, k, v = in_q.get(timeout=30)
            st["recvd"] += 1
            if flag != st["recvd"]:
                raise RuntimeError(f"ring index {i}: flag {flag} != step {st['recvd']}")
            return k, v
        try:
            body(i, send, recv)
        except Exception as exc:  # noqa: BLE001 - reported by the caller
            errors.append(exc)

    threads = [threading.Thread(target=rank, args=(i,)) for i in range(n)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    if errors:
        raise errors[0]


def run_reduce_scatter(xs, dtype: str, op: str, nchannels: int, chunk_elems: int, ring=None):
    """ReduceScatter: xs[r] holds n blocks; rank r gets block r reduced.  Each
    ring index sends the block of its predecessor's rank first, reduces and
    forwards what arrives for n-2 steps, and keeps the last reduction, which
    is its own rank's block.  Messages carry the rank whose block they are."""
    n = len(xs)
    count = xs[0].size // n
    ring = list(range(n)) if ring is None else list(ring)
    ys = [np.zeros(count, dtype=xs[0].dtype) for _ in xs]
    pieces = list(_block_loops(count, ELEM_BYTES[dtype], nchannels, chunk_elems))

    def body(i, send, recv):
        me = ring[i]
        x = xs[me]
        for a, b in pieces:
            def own(q):
                return x[q * count + a:q * count + b]
            if n == 1:
                ys[me][a:b] = own(me)
                continue
            q = ring[(i - 1) % n]
            send(q, own(q))
            for _ in range(n - 2):
                q, v = recv()
                send(q, hop(dtype, hop_op(op), v, own(q)))
            q, v = recv()
            if q != me:
                raise RuntimeError(f"ring index {i} ends with the block of rank {q}")
            fin = hop(dtype, hop_op(op), v, own(q))
            ys[me][a:b] = divide(dtype, fin, n) if op == "avg" else fin
    _threads(n, body)
    return ys


def run_all_gather(xs, dtype: str, nchannels: int, chunk_elems: int, ring=None):
    """AllGather: rank r's output holds every rank's input, block q from rank
    q.  Each ring index copies and sends its own input, then keeps and
    forwards what arrives (n-2 times) and keeps the last one."""
    n = len(xs)
    count = xs[0].size
    ring = list(range(n)) if ring is None else list(ring)
    ys = [np.zeros(n * count, dtype=xs[0].dtype) for _ in xs]
    pieces = list(_block_loops(count, ELEM_BYTES[dtype], nchannels, chunk_elems))

    def body(i, send, recv):
        me = ring[i]
        y = ys[me]
        for a, b in pieces:
            y[me * count + a:me * count + b] = xs[me][a:b]
            if n == 1:
                continue
            send(me, xs[me][a:b])
            for _ in range(n - 2):
                q, v = recv()
                y[q * count + a:q * count + b] = v
                send(q, v)
            q, v = recv()
            y[q * count + a:q * count + b] = v
    _threads(n, body)
    return ys

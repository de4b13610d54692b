"""Brute-force double-binary-tree AllReduce for tiny inputs, written apart
from the C oracle so the two can pin each other.

The tree is built differently from the oracle: only each rank's PARENT is
computed from the bit rule the pages state in words (the lowest set bit is
cleared and the next higher bit set; if that is not a rank, the bit is only
cleared), and every vertex's children are found by inverting that relation.
A child smaller than its parent takes slot 0, a larger one slot 1 (the pages:
"if smaller than the parent, we are his first child, otherwise his second").
Tree 1 renames the ranks of tree 0: mirrored (r <-> n-1-r) for even n,
shifted by one for odd n.

The reduction is a recursion over the tree, evaluated elementwise with the
numpy/torch hop of ``refs.py``: value(v) = x_v folded with value(child 0),
then value(child 1), each as op(received, local).  Channel c uses tree c mod 2
and the channel ranges come from the oracle's pinned partition.  The average
folds like sum and divides the root's value by n once.
"""
from __future__ import annotations

import numpy as np

import oracle
from refs import divide, hop, hop_op


def _btree_parent(n: int, r: int) -> int:
    if r == 0:
        return -1
    b = r & -r                      # lowest set bit
    p = (r & ~b) | (b << 1)
    return p if p < n else (r & ~b)


def tree_links(n: int, t: int):
    """(parent, [slot0 child, slot1 child]) per rank of tree t, -1 = none."""
    if t == 0:
        to_base = from_base = lambda r: r
    elif n % 2 == 0:
        to_base = from_base = lambda r: n - 1 - r
    else:
        to_base = lambda r: (r - 1) % n
        from_base = lambda r: (r + 1) % n
    base_parent = [_btree_parent(n, r) for r in range(n)]
    base_kids = [[-1, -1] for _ in range(n)]
    for r, p in enumerate(base_parent):
        if p >= 0:
            slot = 0 if r < p else 1
            assert base_kids[p][slot] == -1, "two children in one slot"
            base_kids[p][slot] = r
    parent = [-1] * n
    kids = [[-1, -1] for _ in range(n)]
    for v in range(n):
        bv = to_base(v)
        bp = base_parent[bv]
        parent[v] = -1 if bp < 0 else from_base(bp)
        kids[v] = [-1 if k < 0 else from_base(k) for k in base_kids[bv]]
    return parent, kids


def tree_value(xs, dtype: str, op: str, kids, v: int, lo: int, hi: int) -> np.ndarray:
    acc = np.array(xs[v][lo:hi], copy=True)
    for k in kids[v]:
        if k >= 0:
            acc = hop(dtype, hop_op(op), tree_value(xs, dtype, op, kids, k, lo, hi), acc)
    return acc


def run(xs, dtype: str, op: str, nchannels: int):
    """Outputs of the tree AllReduce (all ranks get the root's value)."""
    n = len(xs)
    count = xs[0].size
    out = np.array(xs[0], copy=True)
    if n == 1:
        return [out]
    for c in range(nchannels):
        lo, hi = oracle.channel_range(count, dtype, nchannels, c)
        if hi <= lo:
            continue
        parent, kids = tree_links(n, c % 2)
        root = parent.index(-1)
        val = tree_value(xs, dtype, op, kids, root, lo, hi)
        out[lo:hi] = divide(dtype, val, n) if op == "avg" else val
    return [out.copy() for _ in range(n)]

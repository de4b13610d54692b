"""Where the tree AllReduce's wavefronts wait: a role profile.

Uses a diagnostic build of the library whose Simple tree kernels record,
per wavefront, its first and last wall-clock tick, the ticks its slices
waited for their inputs (the children's, or the parent's on the way down)
and for free output slots, and its role (in the split form, the two halves
of a split role apart).  RINGAR_TREE_SPLIT=0 in the environment profiles
the form with one wavefront a role.  Prints, per kind of role, the
mean over its wavefronts.  The diagnostic build is never the library the
package loads by default.

    python -m ring_allreduce_reduce_amd._build --role-profile /tmp/libringar_roleprof.so
    python ring_allreduce_reduce_amd/examples/tree_role_profile.py /tmp/libringar_roleprof.so
"""
import collections
import ctypes
import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import ring_allreduce_reduce_amd as ra  # noqa: E402


def main(lib_path):
    ra.LIB_PATH = os.path.abspath(lib_path)
    lib = ra.load()
    lib.ringar_role_profile.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    ticks_per_us = 100.0   # the 100 MHz wall clock of MI355X (hipDeviceAttributeWallClockRate)
    dev = torch.device("cuda:0")
    n = 8
    print("tree AllReduce, 8 ranks, fp32 sum, Simple; per kind of role: wavefronts, mean us from its start to "
          "its end (busy), waiting for inputs, waiting for output slots, slices; mean us after the launch's "
          "first start and before its last end")
    for nbytes, nch in ((64 << 20, 32), (64 << 20, 16), (8 << 20, 32)):
        count = nbytes // 4
        xs = [torch.randn(count, device=dev) for _ in range(n)]
        ys = [torch.empty_like(x) for x in xs]
        plan = ra.ringar_plan(count, "float32", n, nch, "Simple", ra.make_config(algo="tree"))
        for _ in range(5):
            ra.allreduce(xs, ys, op="sum", nchannels=nch, proto="Simple", algo="tree")
        torch.cuda.synchronize()
        assert lib.ringar_role_profile(None, 0, 1) == 0
        ra.allreduce(xs, ys, op="sum", nchannels=nch, proto="Simple", algo="tree")
        torch.cuda.synchronize()
        buf = np.zeros((4096, 8), dtype=np.uint64)
        assert lib.ringar_role_profile(buf.ctypes.data, buf.nbytes, 0) == 0
        rows = buf[buf[:, 1] > 0].astype(np.int64)
        t0, t1 = rows[:, 0].min(), rows[:, 1].max()
        form = f"split form, {plan.tree_waves_per_lane} wavefronts per lane" if plan.tree_split else "one wavefront a role"
        print(f"\n{nbytes >> 20} MiB per rank, {nch} channels, {plan.lanes} lanes, chunk {plan.chunk_bytes >> 10} KiB, {form}: "
              f"{len(rows)} wavefronts, first start to last end {(t1 - t0) / ticks_per_us:.1f} us")
        groups = collections.defaultdict(list)
        for r in rows:
            info = int(r[5])
            nk, bc, root = (info >> 16) & 255, (info >> 8) & 255, (info >> 24) & 1
            split, half = (info >> 32) & 1, (info >> 33) & 1
            kind = ("broadcast" if bc else "root" if root else "reduce") + f", {nk} children"
            if split:
                kind += f", half {half}"
            groups[kind].append(((r[1] - r[0]) / ticks_per_us, r[2] / ticks_per_us, r[3] / ticks_per_us, r[4],
                                 (r[0] - t0) / ticks_per_us, (t1 - r[1]) / ticks_per_us))
        print(f"  {'role':22s} {'waves':>6s} {'busy':>8s} {'wait in':>8s} {'wait out':>8s} {'slices':>7s} "
              f"{'start+':>7s} {'end-':>7s}")
        for kind, g in sorted(groups.items()):
            a = np.array(g, dtype=np.float64)
            print(f"  {kind:22s} {len(g):6d} {a[:, 0].mean():8.1f} {a[:, 1].mean():8.1f} {a[:, 2].mean():8.1f} "
                  f"{a[:, 3].mean():7.1f} {a[:, 4].mean():7.1f} {a[:, 5].mean():7.1f}")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))

"""The split tree form's handshake, checked on the host for every rank count
(`tree_split_role` of the kernel's geometry header, compiled for the host
here, on the library's own tree links): along every connection, a producer
that runs as two halves is one whose consumer waits for both tail words, and
a consumer that runs as two halves is one whose producer waits for both head
words; unused input and output slots wait for nothing.  A mismatch would
leave a wavefront waiting for a word nobody writes (the kernel's bounded
wait would end the call with a timeout) or reading a slot before its other
half is written."""
import os
import shutil
import subprocess

import pytest

import ring_allreduce_reduce_amd as ra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ring_allreduce_reduce_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include <cstring>
#include "ring_geometry.h"
using namespace ringar;
int main() {
  int n;
  while (std::scanf("%d", &n) == 1) {
    TreeArgs ta;
    std::memset(&ta, 0, sizeof(ta));
    for (int t = 0; t < 2; t++)
      for (int v = 0; v < n; v++) {
        int p, c0, c1;
        if (std::scanf("%d %d %d", &p, &c0, &c1) != 3) return 1;
        ta.parent[t][v] = (int8_t)p;
        ta.child[t][0][v] = (int8_t)c0;
        ta.child[t][1][v] = (int8_t)c1;
        if (p < 0) ta.root[t] = v;
      }
    for (int t = 0; t < 2; t++)
      for (int v = 0; v < n; v++)
        for (int b = 0; b < 2; b++) {
          if (b && v == ta.root[t]) continue;   // the root's reduce role also broadcasts
          const SplitRole r = tree_split_role(ta, t, v, b == 1);
          std::printf("%d %d %d %d %d %d %d %d %d\n", n, t, v, b, r.my_split, r.in_split[0], r.in_split[1],
                      r.out_split[0], r.out_split[1]);
        }
  }
  return 0;
}
"""


def _hipcc():
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc") and shutil.which("hipcc") is None,
                    reason="needs hipcc to compile the geometry header for the host")
def test_split_handshake_agrees_on_every_connection(tmp_path):
    src = tmp_path / "handshake.hip"
    src.write_text(PROGRAM)
    exe = tmp_path / "handshake"
    r = subprocess.run([_hipcc(), "--offload-arch=gfx950", "-O2", "-std=c++17",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-I", CSRC, "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(src)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    links = {}
    inp = []
    for n in range(2, 65):
        inp.append(str(n))
        for t in (0, 1):
            for v in range(n):
                links[n, t, v] = ra.ringar_tree(n, t, v)
                inp.append("%d %d %d" % links[n, t, v])
    out = subprocess.run([str(exe)], input="\n".join(inp) + "\n", capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    role = {}
    vals = list(map(int, out.stdout.split()))
    for i in range(0, len(vals), 9):
        n, t, v, b, my, i0, i1, o0, o1 = vals[i:i + 9]
        role[n, t, v, b] = (my, (i0, i1), (o0, o1))
    checked = 0
    for n in range(2, 65):
        for t in (0, 1):
            root = next(v for v in range(n) if links[n, t, v][0] < 0)
            waves = 0
            for v in range(n):
                parent, s0, s1 = links[n, t, v]
                kids = [k for k in (s0, s1) if k >= 0]          # child-slot order
                my, ins, outs = role[n, t, v, 0]
                waves += 2 if my else 1
                # unused slots wait for nothing
                for j in range(len(kids), 2):
                    assert ins[j] == 0, (n, t, v)
                    if v == root:
                        assert outs[j] == 0, (n, t, v)
                # up connections: child k's reduce role -> v's reduce role, input slot j
                for j, k in enumerate(kids):
                    kmy, _, kouts = role[n, t, k, 0]
                    assert kmy == ins[j] and kouts == (my, my), (n, t, v, k)
                    checked += 1
                # down connections: v's reduce role (root) or broadcast role -> k's broadcast role
                down_my, _, down_outs = role[n, t, v, 0] if v == root else role[n, t, v, 1]
                for j, k in enumerate(kids):
                    kmy, kins, _ = role[n, t, k, 1]
                    assert kins == (down_my, down_my) and kmy == down_outs[j], (n, t, v, k)
                    checked += 1
                if v != root:
                    bmy, _, bouts = role[n, t, v, 1]
                    waves += 2 if bmy else 1
                    for j in range(len(kids), 2):
                        assert bouts[j] == 0, (n, t, v)
            # the role table's wavefront count is the plan's
            if t == 0:
                waves0 = waves
            else:
                assert waves == waves0, n
        p = ra.ringar_plan(n << 18, "float32", n, 1, "Simple", ra.make_config(algo="tree"))
        if p.tree_split:
            assert p.tree_waves_per_lane == waves0, n
    assert checked == 2 * sum(2 * (n - 1) for n in range(2, 65))

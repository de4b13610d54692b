"""The block mappings of a launch, checked on the host before any GPU run
uses them (`launch_grid` and `block_group` of the kernel's geometry header,
compiled for the host here): for every member count (the ring's n ring
indices, the tree's 2n - 1 roles) and group count, in both the linear and
the XCD-major mapping, every (group, member) pair is taken by exactly one
workgroup of the grid, the extra workgroups of the XCD-major grid (padding
to whole rounds of 8 groups) land on groups past the last, which the kernels
skip, and in the XCD-major mapping all members of a group share one XCD
(workgroup id modulo 8), as the mapping is meant to."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ring_allreduce_reduce_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include <vector>
#include "ring_geometry.h"
using namespace ringar;
int main() {
  long bad = 0, cases = 0;
  for (int members = 1; members <= 129; members++)
    for (int groups = 1; groups <= 70; groups++)
      for (int x = 0; x < 2; x++) {
        const bool xcd = x == 1;
        const int grid = launch_grid(members, groups, xcd);
        std::vector<int> seen((size_t)members * groups, 0), xcd_of(groups, -1);
        int pad = 0;
        for (int b = 0; b < grid; b++) {
          int g, m;
          block_group(b, members, xcd, &g, &m);
          if (m < 0 || m >= members || g < 0) { bad++; continue; }
          if (g >= groups) { pad++; continue; }
          seen[(size_t)g * members + m]++;
          if (xcd) {
            if (xcd_of[g] < 0) xcd_of[g] = b % kXcds;
            else if (xcd_of[g] != b % kXcds) bad++;
          }
        }
        for (int v : seen) if (v != 1) bad++;
        if (!xcd && pad != 0) bad++;
        if (xcd && pad != grid - members * groups) bad++;
        if (xcd && (grid % (kXcds * members) != 0 || grid - members * groups >= kXcds * members)) bad++;
        cases++;
      }
  std::printf("%ld %ld\n", cases, bad);
  return 0;
}
"""


def _hipcc():
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc") and shutil.which("hipcc") is None,
                    reason="needs hipcc to compile the geometry header for the host")
def test_every_block_maps_to_one_rank_channel_lane(tmp_path):
    src = tmp_path / "block_map.hip"
    src.write_text(PROGRAM)
    exe = tmp_path / "block_map"
    r = subprocess.run([_hipcc(), "--offload-arch=gfx950", "-O2", "-std=c++17",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-I", CSRC, "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(src)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    cases, bad = map(int, out.stdout.split())
    assert cases == 129 * 70 * 2 and bad == 0, out.stdout

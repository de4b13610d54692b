"""The int8 reduction ops that the kernels apply to four bytes of a word at
once (`I8::op4`: sum with the carry kept out of each byte's top bit,
products and signed min / max on even and odd bytes as 16-bit lanes) equal
the byte-by-byte ops (`I8::op`, the oracle's definitions: wraparound sum
and product, signed min / max) for every pair of bytes at every byte
position, with varied neighbouring bytes.  The kernel header is compiled for
the host here (no GPU)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ring_allreduce_reduce_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include "ring_kernel_impl.h"
using ringar::I8;
template <int OP> static long check() {
  long bad = 0;
  for (uint32_t x = 0; x < 256; x++)
    for (uint32_t y = 0; y < 256; y++)
      for (int pos = 0; pos < 4; pos++) {
        const uint32_t fa = 0x5a3c81ffu ^ (x * 0x01010101u), fb = 0x7e0080c3u ^ (y * 0x00ff00ffu);
        const uint32_t a = (fa & ~(0xffu << (8 * pos))) | (x << (8 * pos));
        const uint32_t b = (fb & ~(0xffu << (8 * pos))) | (y << (8 * pos));
        const uint32_t r = I8::op4<OP>(a, b);
        for (int k = 0; k < 4; k++) {
          const uint8_t want = I8::op<OP>((uint8_t)(a >> (8 * k)), (uint8_t)(b >> (8 * k)));
          if ((uint8_t)(r >> (8 * k)) != want) bad++;
        }
      }
  return bad;
}
int main() {
  std::printf("%ld %ld %ld %ld %ld\n", check<0>(), check<1>(), check<2>(), check<3>(), check<4>());
  return 0;
}
"""


def _hipcc():
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc") and shutil.which("hipcc") is None,
                    reason="needs hipcc to compile the kernel header for the host")
def test_int8_word_ops_equal_byte_ops(tmp_path):
    src = tmp_path / "i8_word_ops.hip"
    src.write_text(PROGRAM)
    exe = tmp_path / "i8_word_ops"
    r = subprocess.run([_hipcc(), "--offload-arch=gfx950", "-O2", "-std=c++17",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-I", CSRC, "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(src)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split() == ["0"] * 5, out.stdout

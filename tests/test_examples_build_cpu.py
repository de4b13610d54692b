"""The C and HIP examples under ring_allreduce_reduce_amd/examples compile
against the public header and the built library (CPU: compile and link
only; they run on a GPU)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EX = os.path.join(ROOT, "ring_allreduce_reduce_amd", "examples")
PKG = os.path.join(ROOT, "ring_allreduce_reduce_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

needs_hipcc = pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None,
                                 reason="needs hipcc")


@needs_hipcc
@pytest.mark.parametrize("name", ["latency.cpp", "small_calls.cpp"])
def test_c_examples_link_against_the_library(tmp_path, name):
    assert os.path.exists(os.path.join(PKG, "libringar.so")), "build the library first"
    exe = tmp_path / name.split(".")[0]
    r = subprocess.run([HIPCC, "-O2", "-I", os.path.join(ROOT, "include"), "-o", str(exe), os.path.join(EX, name),
                        "-L", PKG, "-lringar", "-Wl,-rpath," + PKG], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]


@needs_hipcc
def test_hop_latency_example_compiles_for_gfx950(tmp_path):
    exe = tmp_path / "hop_latency"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O2", "-Xclang", "-target-feature", "-Xclang",
                        "-packed-fp32-ops", "-o", str(exe), os.path.join(EX, "hop_latency.hip")],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]

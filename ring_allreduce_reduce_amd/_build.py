"""Builds libringar.so (HIP for gfx950) in-tree with hipcc.

Each translation unit compiles in its own hipcc process (in parallel), then
the objects are linked into one shared library next to this file.
"""
from __future__ import annotations

import os
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libringar.so")
_TYPES = ("i8", "i32", "f16", "bf16", "f32", "f64")
SOURCES = ([f"tree_{t}.hip" for t in _TYPES] + [f"ring_kernel_{t}.hip" for t in _TYPES] +
           [f"ring_rs_{t}.hip" for t in _TYPES] + [f"captured_{t}.hip" for t in _TYPES] +
           ["ring_ag.hip", "ring_launch.hip", "ringar.cpp"])

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fno-gpu-flush-denormals-to-zero",
    # no packed fp32 instructions: plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(out: str = LIB, extra: list | None = None, verbose: bool = False, jobs: int = 8) -> str:
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory(prefix="ringar_build_") as tmp:
        def compile_one(src: str) -> str:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            cmd = [_hipcc(), *HIPCC_FLAGS, *(extra or []), *inc, "-x", "hip", "-c",
                   os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
            return obj

        with ThreadPoolExecutor(max_workers=jobs) as pool:
            objs = list(pool.map(compile_one, SOURCES))
        link = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out + ".tmp"]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    import sys
    if len(sys.argv) == 3 and sys.argv[1] == "--role-profile":
        # a diagnostic build: the tree kernels record where each wavefront
        # waited (never the library the package loads)
        print(build(out=os.path.abspath(sys.argv[2]), extra=["-DRINGAR_ROLE_PROFILE"]))
    else:
        build(verbose=False)
        print(LIB)

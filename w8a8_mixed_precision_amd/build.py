"""Build libw8mp.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m w8a8_mixed_precision_amd.build

Every source is compiled every time this runs. First the host program
csrc/gelu_table_gen.cpp is built and run: it writes the GELU tables that the
kernels include (gelu_table.inc, in the build's temporary folder). Then one
hipcc process per HIP source (in parallel), then one link.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libw8mp.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions (v_pk_*_f32) in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _jobs() -> int:
    for var in ("MAX_JOBS", "CMAKE_BUILD_PARALLEL_LEVEL"):
        v = os.environ.get(var, "")
        if v.isdigit() and int(v) > 0:
            return min(int(v), 16)
    return min(os.cpu_count() or 4, 16)


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="w8mp_build_") as tmpdir:
        gen = os.path.join(tmpdir, "gelu_table_gen")
        cmd = [CXX, "-O2", "-std=c++17", os.path.join(PKG, "csrc", "gelu_table_gen.cpp"), "-o", gen]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        subprocess.run([gen, os.path.join(tmpdir, "gelu_table.inc")], check=True)
        inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"), "-I", tmpdir]
        def compile_one(src: str) -> str:
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            cmd = [HIPCC, *FLAGS, *inc, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
            return obj

        srcs = sources()
        with cf.ThreadPoolExecutor(max_workers=_jobs()) as ex:
            objs = list(ex.map(compile_one, srcs))
        tmp = LIB + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
    sys.exit(0)

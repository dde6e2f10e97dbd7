"""Build libmoedecode.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "libmoedecode.so")
SOURCES = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from emitting packed FP32 VALU ops.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-command-line-argument",
         "-I", os.path.join(ROOT, "include")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")


def build_library(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every csrc/*.hip to an object (in parallel), then link the shared library."""
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 16)
    tmpdir = tempfile.mkdtemp(prefix="moed_build_")
    try:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in SOURCES]
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            list(ex.map(lambda so: _run([HIPCC, *FLAGS, "-c", so[0], "-o", so[1]], verbose),
                        zip(SOURCES, objs)))
        tmp = LIB_PATH + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
        os.replace(tmp, LIB_PATH)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))

"""Builds librlscan.so (HIP, gfx950) in the package directory.

Usage:  python -m linear_recurrence_scan_coefficient_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "librlscan.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
# one translation unit per estimator plus the host part, compiled in parallel
SOURCES = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
HEADERS = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hpp")) + [
    os.path.join(INCLUDE, "rlscan.h")]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    # keep the compiler from emitting packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(out: str = LIB_PATH, extra_flags=(), verbose: bool = False, jobs: int = 0) -> str:
    """Compiles every translation unit to an object (in parallel), then links
    the shared library."""
    import concurrent.futures
    import tempfile
    jobs = jobs or min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with tempfile.TemporaryDirectory(prefix="rlscan_build_") as tmpdir:
        def compile_one(src):
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, "-c", src,
                   "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
            return obj
        with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
            objs = list(pool.map(compile_one, SOURCES))
        tmp = out + ".tmp"
        cmd = [hipcc(), "--offload-arch=gfx950", "-fPIC", "-shared", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def is_stale(path: str = LIB_PATH) -> bool:
    if not os.path.exists(path):
        return True
    t = os.path.getmtime(path)
    return any(os.path.getmtime(f) > t for f in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)

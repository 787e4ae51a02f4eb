"""Compile the HIP library for gfx950 in-tree (hipcc, no GPU needed).

Each translation unit is compiled to an object in its own hipcc process (in
parallel), then the objects are linked into ``librans_hip.so``.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "librans_hip.so")
SOURCES = ["rans_prep.hip", "rans_encode.hip", "rans_decode.hip", "rans_tables.hip", "rans_latent.hip",
           "rans_interleaved.hip", "rans_noalloc.hip", "rans_abi.hip"]
ARCH = os.environ.get("RANS_HIP_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 instructions stay off: only the compiler's scalar forms are used
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _jobs() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16, len(SOURCES)))


def build(verbose: bool = False, extra=()) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    with tempfile.TemporaryDirectory(prefix="rans_build_") as tmpdir:
        def compile_one(src):
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            cmd = ["hipcc", *FLAGS, "-I", INCLUDE, "-I", CSRC, *extra, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
            return obj

        with ThreadPoolExecutor(max_workers=_jobs()) as ex:
            objs = list(ex.map(compile_one, srcs))
        tmp = f"{LIBRARY}.tmp{os.getpid()}"
        cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

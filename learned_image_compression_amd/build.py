"""Compile the HIP library for gfx950 in-tree (hipcc, no GPU needed)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "librans_hip.so")
SOURCES = ["rans_prep.hip", "rans_encode.hip", "rans_decode.hip", "rans_tables.hip", "rans_latent.hip",
           "rans_interleaved.hip", "rans_abi.hip"]
ARCH = os.environ.get("RANS_HIP_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # packed fp32 instructions stay off: only the compiler's scalar forms are used
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False, extra=()) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = f"{LIBRARY}.tmp{os.getpid()}"
    cmd = ["hipcc", *FLAGS, "-I", INCLUDE, "-I", CSRC, *extra, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build libkvq.so (the C-ABI codec library) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
SOURCES = ["kvq_host.cpp", "kvq_encode.hip", "kvq_decode.hip", "kvq_score.hip", "kvq_pca.hip",
           "kvq_misc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed f32 VALU instructions are disabled for all device code: the plain f32 forms are used.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fno-gpu-rdc", "-munsafe-fp-atomics"]


def build(verbose: bool = False) -> str:
    srcs = []
    for s in SOURCES:
        p = os.path.join(CSRC, s)
        srcs += (["-x", "hip", p] if s.endswith(".cpp") else [p])
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build libkvq.so (the C-ABI codec library) for gfx950 with hipcc, in-tree.

Each source compiles to an object in parallel; the objects are then linked into one shared
library next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
OBJ = os.path.join(HERE, "_obj")
SOURCES = ["kvq_host.cpp", "kvq_encode.hip", "kvq_encode_mx.hip", "kvq_encode_kron.hip",
           "kvq_decode.hip",
           "kvq_decode_h.hip", "kvq_score.hip", "kvq_pca.hip", "kvq_misc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed f32 VALU instructions are disabled for all device code: the plain f32 forms are used.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-gpu-rdc"]


# Per-source extras. The matrix-core kernels keep MFMA results in architectural VGPRs: the
# quantiser or the softmax reads every one of them (accumulator registers would cost a move
# each), and the unified register file then holds two attention waves per SIMD.
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]
EXTRA = {"kvq_encode_mx.hip": _VGPR_FORM, "kvq_encode_kron.hip": _VGPR_FORM, "kvq_decode_h.hip": _VGPR_FORM, "kvq_score.hip": _VGPR_FORM}


def _compile(src: str, verbose: bool) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + EXTRA.get(src, []) + ["-c"] + \
          (["-x", "hip"] if src.endswith(".cpp") else []) + [path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    workers = min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

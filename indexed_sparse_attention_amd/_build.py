"""Build libdsa.so (the C-ABI library) with hipcc for gfx950, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdsa.so")
SOURCES = ["index_score.hip", "topk.hip", "sparse_mla.hip", "noalloc_ws.hip", "dsa_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-variable",
    "-Wno-unused-function",
    # keep the compiler from emitting packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-source flags.  The indexer's matrix-core kernels apply ReLU and the head
# weights to every MFMA result; with the results in accumulation registers each
# element costs one more copy instruction (v_accvgpr_read) before the VALU can
# use it, so that file takes the MFMA forms that write arithmetic registers.
# (The attention kernel keeps its 128 output accumulators in accumulation
# registers on purpose, so the option is not global.)
EXTRA = {"index_score.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"]}
OBJ_DIR = os.path.join(HERE, "_build")


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libdsa.so (always recompiles)."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = []
    for s in SOURCES:
        obj = os.path.join(OBJ_DIR, os.path.splitext(s)[0] + ".o")
        cmd = [HIPCC, *FLAGS, *EXTRA.get(s, []), "-c", os.path.join(CSRC, s), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

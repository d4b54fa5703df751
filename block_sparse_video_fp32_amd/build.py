"""Build step: compile the HIP kernels and the C-ABI host layer for gfx950
into ``libsparse_attn.so`` next to this file (in-tree, no JIT cache).

    python -m block_sparse_video_fp32_amd.build
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libsparse_attn.so")

SOURCES = ["sparse_attn_kernels.hip", "dense_attend_kernels.hip", "reblock_kernels.hip", "sparse_attn_noalloc.hip",
           "sparse_attn_api.cpp"]

# Packed fp32 instructions are switched off for all device code.
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source and link the shared library; returns its path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = OUT + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if verbose and res.stderr.strip():
        sys.stderr.write(res.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))

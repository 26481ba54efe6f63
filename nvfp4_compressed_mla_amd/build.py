"""Build the HIP library ``libmla_nvfp4.so`` in-tree for gfx950 with hipcc.

Usage: ``python -m nvfp4_compressed_mla_amd.build`` (also called by ``__graft_entry__.build()``).
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmla_nvfp4.so")
SOURCES = ["api.hip", "codec.hip", "decode.hip", "fp8.hip", "indexer.hip", "layout.hip", "topk.hip", "union.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed FP32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # keep MFMA accumulators in VGPRs: the softmax rescale multiplies them with VALU, and an
    # AGPR home for them costs a full AGPR<->VGPR copy of the output tile on every iteration
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

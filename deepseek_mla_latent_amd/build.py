"""Build ``libmla_latent.so`` in-tree with hipcc for gfx950.

``python -m deepseek_mla_latent_amd.build`` (or ``__graft_entry__.build()``) compiles every HIP
source under ``csrc/`` into one shared library next to this file.  Always recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_NAME = "libmla_latent.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["mla_api.cpp", "decode_attn.hip", "projections.hip", "prefill.hip", "prepare.hip", "fp8.hip",
           "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# gfx950 only; packed-fp32 VALU ops are disabled (plain fp32 code is scalar fp32).  The attention
# kernel's MFMA stream is written as fully unrolled loops whose bodies exceed the default size
# limit of "#pragma unroll"; partially unrolled, its register arrays would be indexed at run time.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-pragma-unroll-threshold=1000000",
    "-Wall", "-Wno-unused-result",
]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build ``libmla_latent.so`` in-tree with hipcc for gfx950.

``python -m deepseek_mla_latent_amd.build`` (or ``__graft_entry__.build()``) compiles every HIP
source under ``csrc/`` into one shared library next to this file, and the same sources with
``MLA_DEBUG_BOUNDS`` into ``libmla_latent_debug.so`` (page-table checks on the device).  Always
recompiles.
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
# The same sources with MLA_DEBUG_BOUNDS: the kernels check the page table on the device.
DEBUG_LIB_PATH = os.path.join(PKG, "libmla_latent_debug.so")
SOURCES = ["mla_api.cpp", "decode_attn.hip", "projections.hip", "prefill.hip", "prepare.hip", "fp8.hip",
           "noalloc.hip", "debug_bounds.hip"]
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


def _compile(out_path: str, extra, verbose: bool) -> subprocess.Popen:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    cmd = [HIPCC, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", out_path + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def build(verbose: bool = False) -> str:
    """Compile the library and its bounds-checked variant (in parallel); return the library's path."""
    jobs = [(LIB_PATH, _compile(LIB_PATH, [], verbose)),
            (DEBUG_LIB_PATH, _compile(DEBUG_LIB_PATH, ["-DMLA_DEBUG_BOUNDS"], verbose))]
    failed = []
    for path, proc in jobs:
        log, _ = proc.communicate()
        out = "\n".join(l for l in log.splitlines() if "packed-fp32-ops" not in l)
        if proc.returncode != 0:
            failed.append(f"hipcc failed for {os.path.basename(path)} ({proc.returncode}):\n{out}")
        elif verbose and out.strip():
            print(out)
    if failed:
        raise RuntimeError("\n".join(failed))
    for path, _ in jobs:
        os.replace(path + ".tmp", path)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

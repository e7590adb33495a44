"""Build libsge.so (HIP for gfx950) in-tree with hipcc.

Usage: ``python -m scaled_gemm_epilogues_amd.build`` (or ``__graft_entry__.build()``).
Compiles every source under ``csrc/`` and links ``scaled_gemm_epilogues_amd/libsge.so``.
"""

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsge.so")
SOURCES = ["gemm.hip", "quant.hip", "aux.hip", "norm.hip", "abi.cpp"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # Keep the compiler from forming packed fp32 (v_pk_*_f32) instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Every `#pragma unroll` loop here is meant to unroll fully (the accumulator tiles are indexed
    # by its counters); the default size cap left the clamped dSwiGLU epilogue's pass loop rolled,
    # which put the MXFP8 tile's accumulators in scratch.
    "-mllvm", "-pragma-unroll-threshold=65536",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if c == "hipcc" or os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src):
    out = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    return out


def build(verbose=False):
    os.makedirs(OBJ, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

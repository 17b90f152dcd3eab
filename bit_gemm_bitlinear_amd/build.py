"""Builds libbitlinear.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m bit_gemm_bitlinear_amd.build

Every source is compiled with hipcc for gfx950 only.  Float code is compiled
with contraction into FMAs off and IEEE division (hipcc's default), so the
kernels' fp32 steps are single correctly rounded operations.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libbitlinear.so")
SOURCES = ["abi.hip", "act_quant.hip", "decode.hip", "decode_fused.hip", "prefill.hip", "pack.hip"]
# measurement kernels (include/bitlinear_probes.h), a library of their own
PROBE_LIB = os.path.join(PKG, "libbitlinear_probes.so")
PROBE_SOURCES = ["probes.hip"]
ARCH = "gfx950"

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-ffp-contract=off", "-Wall", "-Wno-unused-function",
    # keep the compiler from forming packed fp32 ops on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libbitlinear.so")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libbitlinear.so and
    libbitlinear_probes.so; returns the path of libbitlinear.so."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        _run([cc, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + len(PROBE_SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES + PROBE_SOURCES))
    for lib, n0, n1 in ((LIB, 0, len(SOURCES)), (PROBE_LIB, len(SOURCES), len(objs))):
        tmp = lib + ".tmp"
        _run([cc, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs[n0:n1]])
        os.replace(tmp, lib)
        if verbose:
            print(f"built {lib}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

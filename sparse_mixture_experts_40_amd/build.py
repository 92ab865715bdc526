"""Build the gfx950 HIP library ``libmoe.so`` in-tree with hipcc.

    python -m sparse_mixture_experts_40_amd.build
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(PKG, "libmoe.so")
ARCH = "gfx950"

# -packed-fp32-ops off: hipcc -O3 must not form packed fp32 ops by itself.
# amdgpu-mfma-vgpr-form: MFMA accumulators in ordinary VGPRs. Kernels with one
# wave per SIMD may use 512 registers, and with inline asm in them the compiler
# otherwise picks the AGPR form, whose results then cost a v_accvgpr move per
# element before any VALU use (the 4-bit fold reads every accumulator).
HIP_FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form",
             "-Wall", "-Wno-unused-result", "-Wno-unused-function"]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["hipcc", *HIP_FLAGS, "-I", os.path.join(os.path.dirname(PKG), "include"),
           *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the gfx target feature; that warning is harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Compile the q4skinny HIP library for gfx950 into this package directory.

    python -m bit_dequant_skinny_amd.build

Produces ``bit_dequant_skinny_amd/libq4skinny.so`` with hipcc.  All device code
is built with packed-fp32 instructions disabled (the compiler still emits
ordinary v_fma_f32 / v_mul_f32) and without floating-point contraction.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libq4skinny.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    # every multiply and add rounds as written: the kernels spell out their
    # fused multiply-adds with fmaf, and the dequantize must round the fp32
    # product before narrowing it (contraction would fold both into one
    # mixed-precision fma with a single rounding and lose the sign of zero)
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results land in ordinary VGPRs, so the fp32 epilogues that
    # scale them (absmax per block) read them without v_accvgpr_read copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False, extra_flags=None) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, *HIPCC_FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC, *sources(),
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device feature flag; that warning is harmless.
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("hipcc failed with status %d" % res.returncode)
    if out.strip() and verbose:
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

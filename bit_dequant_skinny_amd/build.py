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


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device feature flag; that warning is harmless.
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    return res.returncode, out


def build(verbose: bool = False, extra_flags=None, jobs: int = 0) -> str:
    """Compiles every source to an object in parallel (one hipcc per file),
    then links the shared library."""
    from concurrent.futures import ThreadPoolExecutor
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    srcs = sources()
    tag = "%d" % os.getpid()
    objs = [os.path.join(objdir, os.path.basename(src) + "." + tag + ".o") for src in srcs]
    cmds = [[hipcc, *compile_flags, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC, "-c", src,
             "-o", obj] for src, obj in zip(srcs, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    n = jobs or min(len(cmds), max(1, (os.cpu_count() or 1)), 16)
    with ThreadPoolExecutor(max_workers=n) as ex:
        results = list(ex.map(_run, cmds))
    failed = [(c, out) for c, (rc, out) in zip(cmds, results) if rc != 0]
    if failed:
        for c, out in failed:
            sys.stderr.write(" ".join(c) + "\n" + out + "\n")
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
        raise RuntimeError("hipcc failed on %d source(s)" % len(failed))
    tmp = LIB + ".tmp" + tag
    rc, out = _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp])
    for o in objs:
        os.remove(o)
    if rc != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("hipcc link failed with status %d" % rc)
    if out.strip() and verbose:
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

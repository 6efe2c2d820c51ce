"""Build libnvfp4act.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python nvfp4_activation_quantization_amd/build.py   (a plain script: the package itself
       refuses to import until the library exists)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libnvfp4act.so")
SOURCES = ["quantize.hip", "rms_adaln.hip", "swiglu.hip", "residual_rms.hip", "rms_silu.hip", "ln_fp8.hip", "abi.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    # IEEE fp32: no contraction of a*b+c into FMA (the kernels call fmaf where the
    # specification has a fused multiply-add), correctly rounded divide and sqrt, denormals
    # kept (the HIP defaults for gfx950, restated).
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # no packed-FP32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libnvfp4act.so)")


def _run(cmd):
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so: harmless
    noise = "not a recognized feature for this target"
    err = "\n".join(l for l in proc.stderr.splitlines() if noise not in l)
    return proc.returncode, err


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libnvfp4act.so (always rebuilds).  The sources are
    compiled to objects in parallel, then linked."""
    from concurrent.futures import ThreadPoolExecutor
    tag = "%d" % os.getpid()
    objs = [os.path.join(PKG, "_obj_%s_%s.o" % (os.path.splitext(s)[0], tag)) for s in SOURCES]
    cmds = [[hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj] for src, obj in zip(SOURCES, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    try:
        with ThreadPoolExecutor(len(cmds)) as ex:
            results = list(ex.map(_run, cmds))
        for (rc, err), src in zip(results, SOURCES):
            if rc != 0:
                raise RuntimeError("hipcc failed on %s:\n%s" % (src, err))
            if err.strip() and verbose:
                print(err, file=sys.stderr)
        tmp = LIB + ".tmp" + tag
        rc, err = _run([hipcc(), *HIPCC_FLAGS, "-shared", *objs, "-o", tmp])
        if rc != 0:
            raise RuntimeError("hipcc link failed:\n" + err)
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

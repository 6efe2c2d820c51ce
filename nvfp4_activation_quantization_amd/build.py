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
# diagnostics beside the product library (conversion sweeps, the bare-traffic stream): loaded
# by the tests and the benchmark only
SELFTEST_LIB = os.path.join(PKG, "libnvfp4act_selftest.so")
SELFTEST_SOURCES = ["selftest.hip"]

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


def source_digest() -> str:
    """sha256 over csrc/* and include/nvfp4act.h in name order, each file preceded by its
    name; compiled into the library (nvfp4act_source_digest) and checked by the binding."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(CSRC, "*"))) + [os.path.join(ROOT, "include", "nvfp4act.h")]:
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def generate_tables(tag: str) -> str:
    """Compile and run silu_tables_gen (host C++) into _build/: the bf16 and fp16 SiLU tables
    the kernels include.  Raises if the generator fails (an entry fp64 cannot decide)."""
    gen_dir = os.path.join(ROOT, "_build")
    os.makedirs(gen_dir, exist_ok=True)
    exe = os.path.join(gen_dir, "silu_tables_gen_%s" % tag)
    rc, err = _run(["g++", "-O2", "-std=c++17", os.path.join(CSRC, "silu_tables_gen.cpp"), "-o", exe])
    if rc != 0:
        raise RuntimeError("g++ failed on silu_tables_gen.cpp:\n" + err)
    try:
        rc, err = _run([exe, os.path.join(gen_dir, "silu_bf16.inc"), os.path.join(gen_dir, "silu_f16.inc")])
    finally:
        os.remove(exe)
    if rc != 0:
        raise RuntimeError("silu_tables_gen failed:\n" + err)
    return gen_dir


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libnvfp4act.so (always rebuilds).  The sources are
    compiled to objects in parallel, then linked."""
    from concurrent.futures import ThreadPoolExecutor
    tag = "%d" % os.getpid()
    digest = '-DNVFP4ACT_SOURCE_DIGEST="%s"' % source_digest()
    gen_dir = generate_tables(tag)
    all_sources = SOURCES + SELFTEST_SOURCES
    objs = [os.path.join(PKG, "_obj_%s_%s.o" % (os.path.splitext(s)[0], tag)) for s in all_sources]
    cmds = [[hipcc(), *HIPCC_FLAGS, "-I", gen_dir, *([digest] if src == "abi.cpp" else []), "-c",
             os.path.join(CSRC, src), "-o", obj] for src, obj in zip(all_sources, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    try:
        with ThreadPoolExecutor(len(cmds)) as ex:
            results = list(ex.map(_run, cmds))
        for (rc, err), src in zip(results, all_sources):
            if rc != 0:
                raise RuntimeError("hipcc failed on %s:\n%s" % (src, err))
            if err.strip() and verbose:
                print(err, file=sys.stderr)
        n = len(SOURCES)
        for lib, lib_objs in ((LIB, objs[:n]), (SELFTEST_LIB, objs[n:])):
            tmp = lib + ".tmp" + tag
            rc, err = _run([hipcc(), *HIPCC_FLAGS, "-shared", *lib_objs, "-o", tmp])
            if rc != 0:
                raise RuntimeError("hipcc link failed:\n" + err)
            os.replace(tmp, lib)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

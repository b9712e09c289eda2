"""Builds the HIP library libopd_mi355x.so in-tree with hipcc for gfx950.

    python -m draft_model_distillation_amd.build

The library links only the HIP runtime (every kernel, the matrix products of the lm_head-fused path
included, is the library's own); the Python binding loads it with ctypes.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIBNAME = "libopd_mi355x.so"
SOURCES = ["opd_kernels.hip", "opd_epilogue.hip", "opd_sample.hip", "opd_noalloc.hip", "opd_gemm.hip", "opd_api.cpp",
           "opd_pack.cpp", "opd_lmhead.cpp"]
# Row kernels only: the VALU runs with the IEEE mode bit clear, so max/min need no NaN-quieting
# canonicalisation of their operands (inputs are finite by contract). The host file keeps IEEE NaN
# semantics for its argument checks, and the epilogue file the device library's accurate exp/log.
KERNEL_ONLY = ["-fno-honor-nans", "-mno-amdgpu-ieee"]
IEEE_OFF_SOURCES = {"opd_kernels.hip"}

COMMON = [
    "--offload-arch=gfx950",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-ffp-contract=off",
    # packed fp32 VALU forms are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def lib_path() -> str:
    return os.path.join(LIBDIR, LIBNAME)


def build(verbose: bool = False) -> str:
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        if src in IEEE_OFF_SOURCES:
            lang += KERNEL_ONLY
        cmd = [cc, *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        objs.append(obj)
    out = lib_path()
    tmp = out + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-L/opt/rocm/lib",
           "-Wl,-rpath,/opt/rocm/lib", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

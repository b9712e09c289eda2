"""AddressSanitizer + UndefinedBehaviorSanitizer build of the library's host code.

    python -m draft_model_distillation_amd.build_sanitized

The host sources (argument checks, launch planning, exchange-flag bookkeeping, the packer, the
matrix-product planning) are compiled with g++ and both sanitizers; the device code is taken unchanged from the
regular build's objects. The result is a separate library under ``_build/sanitized/`` that the CPU
tests load in a child process (with the sanitizer runtimes preloaded into Python) in place of the
regular one; device code is never instrumented.
"""

from __future__ import annotations

import os
import subprocess
import sys

from . import build as _build

HOST_SOURCES = ["opd_api.cpp", "opd_pack.cpp", "opd_lmhead.cpp"]
DEVICE_OBJECTS = ["opd_kernels.hip.o", "opd_epilogue.hip.o", "opd_sample.hip.o", "opd_noalloc.hip.o", "opd_gemm.hip.o"]
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
OUT_DIR = os.path.join(_build.PKG, "_build", "sanitized")
LIBNAME = "libopd_mi355x_san.so"


def runtime_preload() -> str:
    """The gcc sanitizer runtimes, for LD_PRELOAD of a process that loads the sanitized library."""
    libs = []
    for name in ("libasan.so", "libubsan.so"):
        r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True, check=True)
        libs.append(r.stdout.strip())
    return ":".join(libs)


def build(verbose: bool = False) -> str:
    objdir = os.path.join(_build.PKG, "_build")
    dev_objs = [os.path.join(objdir, o) for o in DEVICE_OBJECTS]
    if not all(os.path.exists(o) for o in dev_objs):
        _build.build(verbose=verbose)
    os.makedirs(OUT_DIR, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(OUT_DIR, src + ".o")
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", *SAN_FLAGS, "-D__HIP_PLATFORM_AMD__",
               "-I", "/opt/rocm/include", "-I", _build.INCLUDE, "-I", _build.CSRC,
               "-c", os.path.join(_build.CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"g++ failed for {src}:\n{r.stdout}\n{r.stderr}")
        objs.append(obj)
    out = os.path.join(OUT_DIR, LIBNAME)
    cmd = ["g++", "-shared", *SAN_FLAGS, *objs, *dev_objs, "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,/opt/rocm/lib", "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

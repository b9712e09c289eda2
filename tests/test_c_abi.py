"""The C ABI used from plain C: tests/c_abi_check.c is compiled with gcc against include/opd.h and
the built library and run (CPU only: argument checks of the device calls, and the host packer and
capacity estimate)."""

import os
import shutil
import subprocess

import pytest

from draft_model_distillation_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_program_against_the_library(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    if not os.path.exists(B.lib_path()):
        B.build()
    libdir = os.path.dirname(B.lib_path())
    exe = str(tmp_path / "c_abi_check")
    cmd = ["gcc", "-std=c11", "-Wall", "-Werror=implicit-function-declaration", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", os.path.join(ROOT, "tests", "c_abi_check.c"), "-o", exe,
           "-L", libdir, "-lopd_mi355x", f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    lines = out.stdout.splitlines()
    assert lines[0].startswith("workspace ") and int(lines[0].split()[1]) > 0
    assert lines[1].startswith("status OPD_ERR_NULL")
    assert lines[2] == "fwd null z 1"
    assert lines[3].startswith("fwd alpha 5") and "alpha" in lines[3]
    assert lines[4] == "sample null blocks 1"
    # first fit of 8,16,5,9,7,1 under 20 rows: requests 0, 2, 4 (8 + 5 + 7)
    assert lines[5] == "pack 0 n=3 rows=20 sel=0,2,4 off=0,8,13,20"
    assert lines[6] == "cap init 0"
    # EMA with beta 0.5: 4000, then 0.5*4000 + 0.5*2000 = 3000, then 0.5*3000 + 0.5*2001 = 2500.5
    assert lines[7] == "cap 4000 3000 2500"
    assert lines[8] == "cap bad beta 5"

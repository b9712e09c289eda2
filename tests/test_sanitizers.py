"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The host sources are rebuilt with both sanitizers (draft_model_distillation_amd.build_sanitized;
device code unchanged), then:
  * tests/c_abi_check.c, compiled with the sanitizers, runs against that library;
  * the ABI, packer and binding-validation tests run in a child Python process that preloads the
    sanitizer runtimes and loads the sanitized library in place of the regular one.
Any report from either sanitizer aborts the program, which fails the test.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1", "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


@pytest.fixture(scope="module")
def san_lib():
    if shutil.which("gcc") is None or shutil.which("g++") is None:
        pytest.skip("gcc / g++ not available")
    from draft_model_distillation_amd import build_sanitized as S

    return S.build(), S.runtime_preload()


def test_c_program_under_sanitizers(san_lib, tmp_path):
    lib, _ = san_lib
    libdir = os.path.dirname(lib)
    name = os.path.basename(lib)[3:-3]
    exe = str(tmp_path / "c_abi_check_san")
    cmd = ["gcc", "-std=c11", "-Wall", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
           os.path.join(ROOT, "tests", "c_abi_check.c"), "-o", exe, "-L", libdir, f"-l{name}",
           f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=dict(os.environ, **SAN_ENV))
    assert out.returncode == 0, out.stdout + out.stderr
    assert "ERROR: AddressSanitizer" not in out.stderr and "runtime error" not in out.stderr
    assert out.stdout.splitlines()[-1] == "cap bad beta 5"


def test_python_abi_tests_under_sanitizers(san_lib):
    lib, preload = san_lib
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=preload, OPD_MI355X_LIB=lib)
    tests = [os.path.join(ROOT, "tests", t) for t in ("test_abi.py", "test_packer.py", "test_binding_validation.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *tests],
                       capture_output=True, text=True, timeout=900, env=env, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
    assert " passed" in r.stdout

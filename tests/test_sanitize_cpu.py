"""Host builds under AddressSanitizer and UndefinedBehaviorSanitizer.

sanitize_oracle.c drives every oracle entry point over exact-size buffers
with special values in the inputs; sanitize_api.cpp drives the C ABI's
argument validation (iq_api.cpp) against recording stand-ins for the kernel
launchers, legal and illegal arguments alike.  A sanitizer report aborts the
program and fails the test.  Both build with the host compilers only: no
device code is compiled or run here.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined,float-cast-overflow",
       "-fno-sanitize-recover=all"]
ENV = {**os.environ, "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0", "UBSAN_OPTIONS": "print_stacktrace=1"}


def build_and_run(cmd, exe):
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert r.stdout.startswith("ok"), r.stdout
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "sanitize_oracle")
    out = build_and_run(["gcc", *SAN, "-std=c11", "-ffp-contract=off", "-o", exe,
                         os.path.join(HERE, "sanitize_oracle.c"), os.path.join(ROOT, "oracle", "iq_oracle.c"), "-lm"],
                        exe)
    assert int(out.split()[1]) > 500


def test_abi_validation_under_sanitizers(tmp_path):
    if shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the HIP headers not available")
    exe = str(tmp_path / "sanitize_api")
    out = build_and_run(["g++", *SAN, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                         "-I", "/opt/rocm/include", "-o", exe, os.path.join(HERE, "sanitize_api.cpp"),
                         os.path.join(ROOT, "int_quantization_amd", "csrc", "iq_api.cpp")], exe)
    assert int(out.split()[1]) > 500

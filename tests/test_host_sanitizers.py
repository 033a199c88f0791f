"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/sanitize/host_driver.cpp drives the encoders (Tiled-CSL on several tile shapes, bitmap,
three-level), import validation of valid and invalid encodings, the handle life cycle,
argument errors and the allocation-failure hook (LSCD_TEST_FAIL_ALLOC) through the C ABI.
It is built with g++ from the library's host sources (lscd_pack.cpp, lscd_api.cpp) and
tests/sanitize/hip_host_stub.cpp, which stands in for the HIP runtime and the kernel launch
tables with host memory and launches that report an error.  Any sanitizer report, leak or
failed check makes the driver exit non-zero.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "unstructured_sparse_skinny_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_host_code_is_sanitizer_clean(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not installed")
    exe = str(tmp_path / "lscd_host_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "lscd_pack.cpp"), os.path.join(CSRC, "lscd_api.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "hip_host_stub.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"), "-pthread", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.stdout[-2000:], r.stderr[-6000:])

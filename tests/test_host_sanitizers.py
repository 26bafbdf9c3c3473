"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

mx_api.cpp (argument validation, plane sizes, dispatch) and mx_grid.cpp
(launch geometry) are compiled for the host with the sanitizers and linked
against stub launchers (tests/host/mx_api_stubs.cpp) and a C driver
(tests/host/mx_api_driver.c) that takes every MX_ERR_* path, passes
out-of-range enum values as a C caller may, and checks what accepted calls
hand to the launchers. No GPU and no HIP runtime are involved: only g++/gcc
and the HIP headers.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "microscaling_block_quantized_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def test_c_abi_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    gxx, gcc = shutil.which("g++"), shutil.which("gcc")
    hip_inc = "/opt/rocm/include"
    if gxx is None or gcc is None or not os.path.isdir(hip_inc):
        pytest.skip("needs g++, gcc and the HIP headers")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    cxx = [gxx, "-std=c++17", "-Wall", "-Wextra"] + SAN + ["-D__HIP_PLATFORM_AMD__", "-I", hip_inc] + inc
    objs = []
    for src in (os.path.join(CSRC, "mx_api.cpp"), os.path.join(CSRC, "mx_grid.cpp"),
                os.path.join(HOST, "mx_api_stubs.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run(cxx + ["-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        objs.append(obj)
    drv = str(tmp_path / "driver.o")
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic"] + SAN + inc +
                       ["-c", os.path.join(HOST, "mx_api_driver.c"), "-o", drv], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    exe = str(tmp_path / "mx_api_driver")
    r = subprocess.run([gxx] + SAN + objs + [drv, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    # verify_asan_link_order=0: a library the environment preloads may come before the ASan runtime
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mx_api host checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr

"""The oracle and the C ABI's host code (argument validation, workspace
layout, state blobs) built with AddressSanitizer and UndefinedBehaviorSanitizer
and driven through every path that needs no GPU (tests/sanitize/driver.cpp).
CPU only: the kernels are not part of this build."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not (shutil.which("gcc") and shutil.which("g++")):
        pytest.skip("gcc/g++ not available")
    out = tmp_path_factory.mktemp("san")
    ora = str(out / "oracle.o")
    subprocess.run(["gcc", *SAN, "-std=c11", "-ffp-contract=off", "-c", "-o", ora,
                    os.path.join(ROOT, "oracle", "gdn_oracle.c")], check=True)
    exe = str(out / "driver")
    subprocess.run(["g++", *SAN, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-o", exe, os.path.join(ROOT, "tests", "sanitize", "driver.cpp"),
                    os.path.join(ROOT, "gated_deltanet_layer_gdn_amd", "csrc", "gdn_api.cpp"), ora,
                    "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-lpthread"],
                   check=True)
    return exe


def test_host_paths_under_asan_ubsan(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               LSAN_OPTIONS=f"suppressions={os.path.join(ROOT, 'tests', 'sanitize', 'lsan.supp')}")
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
    assert "all checks passed" in r.stdout

"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):
the fp64 oracle's C source on edge-case problems, and the library's host side
(argument validation, workspace layout, the wait-status query) with its
kernel launches stubbed.  Both drivers are built with gcc / g++ and every
sanitizer error stops them (-fno-sanitize-recover=all)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")


def _have(tool):
    return shutil.which(tool) is not None


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=ENV, timeout=300)
    return r


@pytest.mark.skipif(not _have("gcc"), reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_driver"
    b = _run(["gcc", "-std=c11", *SAN, "-fopenmp", "-o", str(exe),
              os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
              os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-lm"], ROOT)
    assert b.returncode == 0, b.stderr
    r = _run([str(exe)], ROOT)
    assert r.returncode == 0 and "ALL OK" in r.stdout, r.stdout + r.stderr


@pytest.mark.skipif(not _have("g++"), reason="g++ not available")
def test_host_abi_under_asan_ubsan(tmp_path):
    exe = tmp_path / "abi_driver"
    b = _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-o", str(exe),
              os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"),
              os.path.join(ROOT, "gated_deltanet_layer_02_amd", "csrc", "gdn_api.cpp")], ROOT)
    assert b.returncode == 0, b.stderr
    r = _run([str(exe)], ROOT)
    assert r.returncode == 0 and "ALL OK" in r.stdout, r.stdout + r.stderr

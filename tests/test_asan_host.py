"""The host side of the C ABI (api.cpp: argument checks, workspace layout,
the choice of launches) under AddressSanitizer, on the CPU: api.cpp is
compiled with g++ -fsanitize=address together with stand-ins for the kernel
launchers and HIP runtime calls (tests/asan/host_stubs.cpp), and
tests/asan/host_checks.py drives every entry point's checks in a subprocess
with libasan preloaded.  A memory error anywhere in that code fails the test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_sampling_verify_spec_amd", "csrc")


def _gxx():
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("g++ not found")
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not asan or not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("libasan not found")
    return gxx, asan


def test_host_checks_under_address_sanitizer(tmp_path):
    gxx, asan = _gxx()
    lib = tmp_path / "libspecverify_asan.so"
    cmd = [gxx, "-std=c++17", "-shared", "-fPIC", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address",
           "-D__HIP_PLATFORM_AMD__", "-D__align__(n)=__attribute__((aligned(n)))", "-DHIP_SYMBOL(x)=(&(x))",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", "/opt/rocm/include",
           os.path.join(CSRC, "api.cpp"), os.path.join(ROOT, "tests", "asan", "host_stubs.cpp"), "-o", str(lib)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "asan", "host_checks.py"), str(lib)],
                       capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0 and "host checks ok" in r.stdout, out[-4000:]

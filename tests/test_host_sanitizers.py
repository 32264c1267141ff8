"""Host build of the C ABI's argument validation (kda_api.cpp) under the
address and undefined-behaviour sanitizers, linked against host-only stand-ins
for the HIP launchers (tests/host_sanitize/stub_launchers.cpp) and driven
through every entry point with valid and invalid arguments
(tests/host_sanitize/abi_driver.cpp).  Any out-of-bounds access, signed
overflow or invalid load aborts the driver; a wrong status code, or a launch
reached by an invalid call, fails it."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_chunkwise_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_sanitize")


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_abi_validation_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "kda_api.cpp"), os.path.join(HERE, "stub_launchers.cpp"),
           os.path.join(HERE, "abi_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "abi driver: ok" in r.stdout

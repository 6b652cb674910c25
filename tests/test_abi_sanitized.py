"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

fa_api.hip (argument checks, workspace layout, launch splitting) is compiled
host-only with both sanitizers and linked with stand-in launchers that record
their arguments and launch nothing (tests/sanitize/abi_stubs.cpp); a driver
(tests/sanitize/abi_driver.cpp) calls every entry point with valid and invalid
arguments, including sizes near the integer limits, and checks the statuses and
that everything handed to the launchers stays inside the caller's buffers. No
GPU and no device code are involved. CPU only.
"""
import os
import subprocess

import pytest

from exact_io_aware_61_amd import build as fab

HERE = os.path.dirname(os.path.abspath(__file__))
SAN = os.path.join(HERE, "sanitize")


def test_c_abi_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    try:
        hipcc = fab.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "abi_driver")
    # host-only compilation; each -fsanitize= applies to the host pass only
    cmd = [hipcc, "--cuda-host-only", "-x", "hip", "-std=c++17", "-O1", "-g",
           "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-I", fab.INCLUDE, "-I", fab.CSRC, "-I", SAN,
           os.path.join(fab.CSRC, "fa_api.hip"), os.path.join(SAN, "abi_stubs.cpp"),
           os.path.join(SAN, "abi_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "all checks passed" in r.stdout, r.stdout + r.stderr[-3000:]

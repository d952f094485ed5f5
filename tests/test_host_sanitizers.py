"""The C ABI's validation and dispatch (dispatch.cpp), built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer against host stand-ins for
the HIP launchers, driven through every entry point (tests/host_sanitize/).
CPU only: no GPU code is built or run."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_dispatch_under_asan_ubsan(tmp_path):
    exe = tmp_path / "abi_driver"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer",
           os.path.join(ROOT, "fp8_weight_only_fp4w_amd", "csrc", "dispatch.cpp"),
           os.path.join(HERE, "host_sanitize", "stub_launchers.cpp"),
           os.path.join(HERE, "host_sanitize", "abi_driver.cpp"), "-o", str(exe)]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.stdout + r.stderr)[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]

"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The CPU oracle, built with g++ and the sanitizers, driven through every
  entry point on small seeded rows with its edge cases
  (tests/native/oracle_sanitize_driver.cpp).
* The host half of the C ABI (csrc/api.cpp: argument checks, workspace
  sizing and layout, segment planning), built host-only with the sanitizers
  and linked with launch stand-ins that check each launch's segment plan and
  that every workspace array it addresses lies inside the caller's workspace
  and apart from the launch's other arrays (tests/native/api_launch_stubs.cpp),
  swept over about 20,000 launches of every entry point
  (tests/native/api_sanitize_driver.cpp).
Any sanitizer report ends a driver with a nonzero status.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-pthread", os.path.join(ROOT, "oracle", "vsel_oracle.cpp"),
                    os.path.join(NATIVE, "oracle_sanitize_driver.cpp"), "-o", exe], check=True, capture_output=True)
    assert "0 failures" in run(exe)


def test_api_host_half_under_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not installed")
    exe = str(tmp_path / "api_driver")
    cmd = [HIPCC, "-O1", "-g", "-std=c++17", "--offload-host-only", "-x", "hip", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-I" + os.path.join(ROOT, "include"),
           os.path.join(ROOT, "vocab_row_reductions_amd", "csrc", "api.cpp"),
           os.path.join(NATIVE, "api_launch_stubs.cpp"), os.path.join(NATIVE, "api_sanitize_driver.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True)
    out = run(exe)
    assert "0 launch failures, 0 call failures" in out, out

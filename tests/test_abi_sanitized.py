"""The host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU).

tests/abi_host_check.cpp links kla_api.cpp with stand-in kernel launchers and
drives every entry point with valid, invalid, overlapping, misaligned, empty
and overflowing arguments, as a C caller would (dtype and status codes as
plain ints, out-of-range ones included).  The sanitizers instrument host code
only; no device code is built."""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_sequence_kla_amd", "csrc")
# every sanitizer flag applies to the host compilation alone
HOST_SANITIZERS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                   "-Xarch_host -fno-sanitize-recover=undefined").split()


def _hipcc():
    path = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return path if os.path.exists(path) else shutil.which("hipcc")


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not found")
def test_abi_host_side_is_sanitizer_clean(tmp_path):
    exe = str(tmp_path / "abi_host_check")
    cmd = [_hipcc(), "-x", "hip", "--offload-host-only", "-O1", "-g", "-std=c++17",
           "-fno-omit-frame-pointer", *HOST_SANITIZERS,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "abi_host_check.cpp"), os.path.join(CSRC, "kla_api.cpp"),
           "-o", exe]
    c = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert c.returncode == 0, c.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and "all checks passed" in r.stdout, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr

"""The host half of the C ABI and the C oracle under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only, gcc). Kernel launchers are stubbed
(tests/sanitize/stub_launch.cpp); the drivers call every host entry point
over shapes, splits and strides at extreme values (INT_MAX, 2^48, LLONG_MAX,
negatives), where the extent arithmetic would overflow if it were not
guarded, and the oracle on small shapes. Any sanitizer report fails the
test (-fno-sanitize-recover)."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="gcc not available")


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"{exe} failed ({r.returncode}):\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    return r.stdout


def test_host_api_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_api_driver")
    srcs = [os.path.join(ROOT, "tests", "sanitize", "host_api_driver.cpp"),
            os.path.join(ROOT, "tests", "sanitize", "stub_launch.cpp"),
            os.path.join(ROOT, "gqa_attention_split_amd", "csrc", "mga_api.cpp")]
    subprocess.run(["g++", "-std=c++17", *SAN, "-o", exe, *srcs], check=True, capture_output=True, text=True)
    out = _run(exe)
    assert "fails: 0" in out, out


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    srcs = [os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), os.path.join(ROOT, "oracle", "gqa_oracle.c")]
    subprocess.run(["gcc", "-std=c11", *SAN, "-o", exe, *srcs, "-lm"], check=True, capture_output=True, text=True)
    out = _run(exe)
    assert "bad=0" in out, out

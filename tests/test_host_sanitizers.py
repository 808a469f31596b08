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


SHAPES = [(2, 256, 4096, 64), (16, 256, 4096, 64), (2, 256, 32768, 64), (64, 8, 8192, 64),
          (128, 256, 16384, 64), (64, 1, 4096, 128), (256, 256, 4096, 64), (8, 256, 8192, 64),
          (4, 100, 1000, 64), (1, 1, 128, 64)]


@pytest.mark.parametrize("cus", [32, 64, 128, 256, 304])
def test_split_policy_fills_the_chip_it_is_given(tmp_path, cus):
    """The split policy at other chip sizes (a compute partition of MI355X, or
    another part): the grid reaches one workgroup per compute unit (two for
    the 32-row shape) with the fewest splits that do so, unless the key count
    runs out of 4-block chunks first; a shape that fills the chip unsplit is
    not split. Runs the host half of the ABI with the device query stubbed."""
    exe = str(tmp_path / "policy_driver")
    srcs = [os.path.join(ROOT, "tests", "sanitize", "policy_driver.cpp"),
            os.path.join(ROOT, "tests", "sanitize", "stub_launch.cpp"),
            os.path.join(ROOT, "gqa_attention_split_amd", "csrc", "mga_api.cpp")]
    subprocess.run(["g++", "-std=c++17", *SAN, "-o", exe, *srcs], check=True, capture_output=True, text=True)
    env = dict(os.environ, MGA_TEST_CUS=str(cus), ASAN_OPTIONS="detect_leaks=1")
    r = subprocess.run([exe, *[",".join(map(str, s)) for s in SHAPES]], capture_output=True, text=True,
                       env=env, timeout=60)
    assert r.returncode == 0, r.stderr
    for line in r.stdout.split("\n"):
        if not line:
            continue
        B, M, N, D, rc, rows, splits = map(int, line.split())
        assert rc == 0
        blocks = -(-N // 128)
        most = max(1, blocks // 4)           # splits that keep 4 key blocks each
        per_cu = 2 if (rows == 32 and D == 64) else 1
        tiles = B * -(-M // rows)
        target = cus * per_cu
        chunk = -(-blocks // splits)
        assert splits == -(-blocks // chunk)  # no empty split
        # the fewest splits that reach the target, unless capped by the key
        # count; the launched count is that request after rounding to equal
        # chunks of whole key blocks
        want = min(-(-target // tiles), most)
        assert tiles * want >= target or want == most, line
        assert -(-blocks // -(-blocks // max(want, 1))) == splits, line

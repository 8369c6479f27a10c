"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only) and driven through every entry point by
tests/pins/sanitize_main.c: seeded finite inputs of every kind the method
meets (zeros, signed zeros, BF16 subnormals, the largest finite BF16, grid
points and midpoints, heavy tails), row lengths from one block to a long
row, ragged group ranges, all three reconstructions, the guided and
global-scale calls, and the rejected-argument paths.  Any out-of-bounds
access, use of uninitialised heap or undefined conversion aborts it."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-ffp-contract=off", "-fno-fast-math",
           "-I", os.path.join(ROOT, "oracle"), os.path.join(ROOT, "oracle", "fp4_oracle.c"),
           os.path.join(ROOT, "tests", "pins", "sanitize_main.c"), "-lm", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "sanitize ok" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])

"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/oracle_asan_check.c drives every oracle entry point (token order,
index with both border rules and per-head shifts, forward and backward with
text tokens, cut tiles, lists one entry too small, invalid arguments); it is
compiled with oracle/sta_oracle.c into one sanitized program that aborts on
the first report.  Its own checks (a permutation, transposed lists holding
the forward lists' pairs, sum dV = sum dO and sum dK = 0) must hold too.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_asan_check")
    subprocess.check_call(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-Wall", "-Wno-unknown-pragmas",
                           os.path.join(ROOT, "oracle", "sta_oracle.c"),
                           os.path.join(ROOT, "tests", "oracle_asan_check.c"), "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle sanitized ok" in r.stdout

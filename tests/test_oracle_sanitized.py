"""The oracle's C code built with AddressSanitizer and UndefinedBehaviorSanitizer (host
only), driven through every dtype, row and key-range form, causal masks, grouped K/V
heads and all rejected arguments by tests/native/oracle_sanitize_driver.c.  Any
out-of-bounds access, leak or undefined operation fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ra_oracle.c")
DRIVER = os.path.join(ROOT, "tests", "native", "oracle_sanitize_driver.c")


def test_oracle_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_sanitized")
    cmd = [gcc, "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           DRIVER, SRC, "-o", exe, "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert "ok" in run.stdout

"""Host code built with AddressSanitizer and UndefinedBehaviorSanitizer (host compilers
only; no GPU code is involved):

* the oracle's C code, driven through every dtype, row and key-range form, causal masks,
  grouped K/V heads and all rejected arguments (tests/native/oracle_sanitize_driver.c);
* the C ABI layer (csrc/ra_api.cpp) against stand-ins for the HIP runtime and the kernel
  launchers (tests/native/abi_stubs.cpp): every entry point with valid arguments must reach
  its launch, with invalid ones must return RA_EINVAL without launching
  (tests/native/abi_sanitize_driver.cpp).

Any out-of-bounds access, leak or undefined operation fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "long_context_exact_ra_amd", "csrc")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=undefined"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _build_and_run(cmd, exe):
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=120)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert "ok" in run.stdout


def test_oracle_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_sanitized")
    _build_and_run([gcc, "-std=c99", "-fopenmp", *SAN,
                    os.path.join(NATIVE, "oracle_sanitize_driver.c"),
                    os.path.join(ROOT, "oracle", "ra_oracle.c"), "-o", exe, "-lm"], exe)


def test_abi_layer_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include/hip"):
        pytest.skip("g++ or the HIP headers not available")
    exe = str(tmp_path / "abi_sanitized")
    _build_and_run([gxx, "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
                    os.path.join(NATIVE, "abi_sanitize_driver.cpp"),
                    os.path.join(NATIVE, "abi_stubs.cpp"), os.path.join(CSRC, "ra_api.cpp"),
                    "-o", exe], exe)

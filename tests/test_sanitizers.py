"""Host sanitizer runs (CPU only): the C oracle and the C ABI's argument
checks built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc/g++,
no recovery), each driven through every function on ragged shapes with
exactly-sized buffers (tests/native/oracle_driver.c) or on boundary-value
argument combinations (tests/native/validate_driver.cpp).  GPU code is not
instrumented."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, env=ENV)
    print(r.stdout[-2000:], r.stderr[-4000:])
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.run(["gcc", *SAN, "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                    os.path.join(ROOT, "oracle", "fp8q_oracle.c"), os.path.join(NATIVE, "oracle_driver.c"),
                    "-o", exe, "-lm"], check=True)
    r = _run([exe])
    assert r.returncode == 0 and "0 failures" in r.stdout


def test_abi_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "validate_driver")
    subprocess.run(["g++", *SAN, "-std=c++17", "-Wall", "-Werror", os.path.join(NATIVE, "validate_driver.cpp"),
                    "-o", exe], check=True)
    r = _run([exe])
    assert r.returncode == 0 and "0 fixed-case failures" in r.stdout

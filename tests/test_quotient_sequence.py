"""The quantizers' division shortcut is IEEE division.

The 1x128, 128x128 and 128x1 kernels form fl32(x / s) as y = RN(x * RN(1/s))
followed by one FMA-based correction (Markstein's step), not with a divide
instruction.  tests/native/quotient_check.c evaluates that sequence with IEEE
fp32 operations on the CPU and compares it with the correctly rounded
quotient bit for bit next to every point where an E4M3 code changes (the
midpoints between consecutive magnitudes and the saturation boundary), for
tens of thousands of tile scales (random, powers of two, around the 2^-64
threshold below which the kernels divide exactly, and at the top of the fp32
range), plus random numerators and signed zeros."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "quotient_check.c")


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("quotient") / "quotient_check")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Werror", SRC,
                    "-o", out, "-lm"], check=True)
    return out


@pytest.mark.parametrize("seed", [1, 2])
def test_fast_quotient_equals_ieee_division(exe, seed):
    r = subprocess.run([exe, "20000", str(seed)], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    n = int(r.stdout.split("checked ")[1].split()[0])
    assert n > 50_000_000

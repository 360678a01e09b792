"""Host check of the kernels' integer division (ia_intdiv.h): the header is
plain integer C++, so g++ compiles the same text the kernels use and
tests/intdiv_check.cpp compares it with exact division: every normalised
reciprocal, the uint8 and uint16 row reciprocals for every row sum below
2^31, edge cases and seeded random pairs. Built with AddressSanitizer and
UndefinedBehaviorSanitizer (any report aborts the run), so signed overflow
or an out-of-range shift in the division fails the test as well."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "integer_only_quantized_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_integer_division_matches_exact_division(tmp_path):
    exe = tmp_path / "intdiv_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-pthread", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I" + CSRC, os.path.join(HERE, "intdiv_check.cpp"),
                    "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0 and res.stdout.strip().endswith("ok"), res.stdout[-2000:]

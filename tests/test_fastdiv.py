"""The two-shot's index arithmetic divides by launch-invariant values (units
per tile, tiles per segment, items per output) with a multiply-high, an add
and a shift (custom_all_reduce_amd/csrc/fastdiv.hpp).  This compiles a small
host program against that header with g++ and checks the quotient against
plain integer division over about 2.2e8 numerator/divisor pairs."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_invariant_divisor_quotient_is_exact(tmp_path):
    exe = tmp_path / "check_fastdiv"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "custom_all_reduce_amd", "csrc"),
                    os.path.join(ROOT, "tests", "fastdiv", "check_fastdiv.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches 0" in r.stdout

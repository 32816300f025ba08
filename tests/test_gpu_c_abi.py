"""The C ABI used from plain C with no PyTorch in the process: the program
tests/c_abi/check_c_abi (built by __graft_entry__.build()) allocates device
buffers with the HIP runtime, runs the one-shot, the reduce-broadcast, the
fused two-shot (explicit and device-kept step ids), LL and LL128 through
include/ar.h and compares every output with the C oracle bit for bit."""
from __future__ import annotations

import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c_abi", "check_c_abi")


def test_c_program_matches_the_oracle():
    if not os.path.exists(BIN):
        pytest.skip(f"{BIN} is not built (__graft_entry__.build() builds it); the Python-side GPU tests "
                    "cover the same calls")
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("c abi ok")
    assert "MISMATCH" not in r.stdout

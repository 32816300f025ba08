"""build() works from sources alone: a copy of the repository's sources with
no built library, oracle or test program builds all three (CPU only; hipcc
cross-compiles for gfx950)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SKIP_DIRS = {".git", "_work", "_build", "gpurun_out", "__pycache__", ".pytest_cache", ".hypothesis", "profiles"}


def test_build_from_a_clean_copy(tmp_path):
    dst = tmp_path / "repo"

    def ignore(d, names):
        out = {n for n in names if n in SKIP_DIRS}
        out |= {n for n in names if n.endswith((".so", ".o")) or n == "check_c_abi"}
        return out

    shutil.copytree(ROOT, dst, ignore=ignore)
    assert not (dst / "custom_all_reduce_amd" / "libar.so").exists()
    r = subprocess.run([sys.executable, "-c", "import __graft_entry__ as g; g.build()"], cwd=dst, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    for built in ("custom_all_reduce_amd/libar.so", "oracle/liboracle.so", "tests/c_abi/check_c_abi"):
        assert (dst / built).exists(), built

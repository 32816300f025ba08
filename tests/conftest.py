import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    """Parse a tests/golden fixture: '#' lines are comments, the rest are whitespace-split rows."""
    rows = []
    with open(os.path.join(ROOT, "tests", "golden", name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def golden_kv(name):
    return {r[0]: r[1] for r in read_golden(name) if len(r) == 2}

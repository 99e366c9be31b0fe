import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def read_golden(name):
    """Parse a golden fixture: '#' comments, then 'KEY v1 v2 ...' lines."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


def read_golden_rows(name, key):
    """Every 'KEY v1 v2 ...' line of a golden fixture with the given key, in
    order (for keys that repeat)."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            parts = line.split()
            if parts and parts[0] == key:
                rows.append(parts[1:])
    return rows


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build(force=False)
    return oracle

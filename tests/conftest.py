import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libvsa.so")


def read_golden(name):
    """Parse a golden fixture: '#' lines are comments; other lines are
    'key v1 v2 ...' (one row per line; repeated keys keep every row)."""
    out = {}
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            out.setdefault(parts[0], parts[1:])
            rows.append(parts)
    return out, rows

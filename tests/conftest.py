import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def golden(name):
    """Parse a tests/golden/*.txt fixture: `key = values` lines, '#' comments,
    ';' separates rows of a matrix."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = [s.strip() for s in line.split("=", 1)]
            rows = [[float(x) for x in r.split()] for r in v.split(";")]
            out[k] = rows if len(rows) > 1 else (rows[0] if len(rows[0]) > 1 else rows[0][0])
    return out

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def read_table(name):
    """Rows of a '|'-separated golden file, comments and blanks skipped."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([c.strip() for c in line.split("|")])
    return rows


def read_figures():
    """key -> (value, printed digits, source) from page_figures.txt."""
    out = {}
    with open(os.path.join(GOLDEN, "page_figures.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, value, digits, source = line.split(None, 3)
            out[key] = (float(value), int(digits), source)
    return out


@pytest.fixture(scope="session")
def figures():
    return read_figures()

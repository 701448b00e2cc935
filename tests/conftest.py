import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def golden_rows(name):
    """Rows of a golden fixture (whitespace-separated, '#' comments skipped)."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip() if not line.lstrip().startswith("#") else ""
            if line:
                rows.append(line.split())
    return rows


@pytest.fixture(scope="session")
def golden():
    return golden_rows

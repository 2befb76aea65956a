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
    """Parse a golden fixture: 'key: values' lines, '#' comments, '|' separates rows.
    Repeated keys accumulate into a list."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            out.setdefault(key.strip(), []).append(val.strip())
    return out


@pytest.fixture
def golden():
    return read_golden

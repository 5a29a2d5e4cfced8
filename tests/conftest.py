import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP library through its C ABI)")


def read_golden(name: str) -> dict:
    """Parse `name = value  # citation` lines of a fixture under tests/golden/."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            out[key] = float(val)
    return out


@pytest.fixture(scope="session")
def page_values():
    return read_golden("page_values.txt")

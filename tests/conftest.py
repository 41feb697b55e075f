import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")
    config.addinivalue_line("markers", "slow: long-running case")


def read_golden(name):
    """Parse a tests/golden fixture: '# comments', 'case X', 'key = numbers'."""
    cases, cur = [], None
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("case "):
                cur = {"name": line[5:].strip()}
                cases.append(cur)
                continue
            if cur is None:
                cur = {"name": "main"}
                cases.append(cur)
            k, v = (p.strip() for p in line.split("=", 1))
            cur[k] = [float(t) for t in v.split()]
    return cases


@pytest.fixture
def golden():
    return read_golden

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU check")


@pytest.fixture(scope="session")
def olib():
    import oracle

    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    return oracle


def load_golden(name):
    """Parse a tests/golden/*.txt fixture: `key = v1 v2 ...` lines, # comments."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            vals = [float(t) for t in v.split()]
            out[k] = vals[0] if len(vals) == 1 else vals
    return out

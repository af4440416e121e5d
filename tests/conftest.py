import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU case")


GOLDEN = os.path.join(ROOT, "tests", "golden")


def read_golden(name):
    """Read a golden text fixture: ``#`` lines are comments (citation and derivation),
    the rest are whitespace-separated integers or floats."""
    vals = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                vals.extend(float(x) if "." in x or "e" in x else int(x) for x in line.split())
    return vals


@pytest.fixture(scope="session")
def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False

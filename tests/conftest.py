import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running")


def read_golden(name):
    """key value pairs from tests/golden/<name>; repeated keys become lists."""
    out = {}
    with open(os.path.join(HERE, "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = line.split(None, 1)
            out.setdefault(key, []).append(float(val))
    return {k: (v[0] if len(v) == 1 else v) for k, v in out.items()}


@pytest.fixture(scope="session")
def golden():
    return read_golden

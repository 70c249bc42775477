import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def golden(key: str):
    """Read one value list from tests/golden/page_values.txt."""
    path = os.path.join(os.path.dirname(__file__), "golden", "page_values.txt")
    with open(path, encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, *vals = line.split()
            if k == key:
                out = [float(v) for v in vals]
                return out[0] if len(out) == 1 else out
    raise KeyError(key)


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle

import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def load_golden(name: str) -> dict:
    """Parse a tests/golden fixture: '# comment' lines, '[name]' headers and
    whitespace-separated numeric rows."""
    out, cur = {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("["):
                cur = line.strip("[]")
                out[cur] = []
                continue
            out[cur].append([float(t) for t in line.split()])
    return {k: np.array(v) for k, v in out.items()}


@pytest.fixture
def golden():
    return load_golden

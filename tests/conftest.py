import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


def read_golden(name):
    """Parse a tests/golden fixture: '#' comments, a bare word opens a section, rows of numbers."""
    sections, cur = {}, None
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            try:
                row = [float(p) for p in parts]
            except ValueError:
                cur = line
                sections[cur] = []
                continue
            sections[cur].append(row)
    import numpy as np
    return {k: np.array(v, dtype=np.float64) for k, v in sections.items()}


@pytest.fixture
def golden():
    return read_golden

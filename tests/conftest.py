import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU oracle runs")


def read_golden(name):
    """Parse a tests/golden text fixture: '# ...' comments, NAME headers, number rows."""
    import numpy as np
    path = os.path.join(ROOT, "tests", "golden", name)
    blocks, cur = {}, None
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line[0].isalpha():
            cur = line
            blocks[cur] = []
        else:
            blocks[cur].append([float(x) for x in line.split()])
    return {k: np.array(v) for k, v in blocks.items()}

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


def load_golden(name):
    """Parse a tests/golden fixture: 'key: v1 v2 ...' lines, '#' comments."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, vals = line.split(":", 1)
            key = key.strip()
            toks = vals.split()
            if key in ("codes", "scales", "res_codes", "res_scales"):
                out[key] = np.array([int(t, 16) for t in toks], np.uint8)
            elif key == "K":
                out[key] = int(toks[0])
            else:
                out[key] = np.array([float(t) for t in toks], np.float32)
    return out


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build()
    return oracle

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def rel_err():
    """Normwise relative error max|x - ref| / max|ref| (0 when both are zero)."""
    import numpy as np

    def f(x, ref):
        x = np.asarray(x, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        den = np.max(np.abs(ref)) if ref.size else 0.0
        num = np.max(np.abs(x - ref)) if ref.size else 0.0
        if den == 0.0:
            return float(num)
        return float(num / den)
    return f

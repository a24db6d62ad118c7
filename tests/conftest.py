import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libgdn.so")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of oracle time)")


def max_rel_err(x, ref):
    """max|x - ref| / max|ref| over a whole tensor, in f64; inf if x has a
    non-finite value where ref is finite."""
    import numpy as np
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    if not np.all(np.isfinite(x)):
        return float("inf")
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(x - ref)) if ref.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


@pytest.fixture(scope="session")
def rel_err():
    return max_rel_err

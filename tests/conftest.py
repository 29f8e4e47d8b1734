import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def to_np(t):
    """torch tensor (any float dtype, any device) -> float64 numpy array of the exact values."""
    return t.detach().to("cpu").double().numpy()


@pytest.fixture
def rng():
    return np.random.default_rng(1234)

import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP library)")
    config.addinivalue_line("markers", "slow: large CPU oracle case")


@pytest.fixture(autouse=True)
def _numpy_errors_raise():
    # the oracle must not silently produce inf/NaN through overflow or 0/0
    with np.errstate(over="raise", invalid="raise", divide="raise"):
        yield

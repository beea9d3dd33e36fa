import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running test")


@pytest.fixture
def rng():
    # a fresh generator per test: a test's inputs do not depend on which
    # tests ran before it in the same process
    import numpy as np
    return np.random.Generator(np.random.PCG64(20261203))

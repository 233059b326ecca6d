import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU work (full-size workloads)")


@pytest.fixture
def rng(request):
    """A generator of its own for every test, seeded from the test's name, so that its
    data do not depend on which tests ran before it (or on the worker under xdist)."""
    import zlib

    import numpy as np
    return np.random.default_rng(zlib.crc32(request.node.nodeid.encode()))

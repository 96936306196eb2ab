import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a ROCm GPU (MI355X / gfx950)")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle._load()  # builds liboracle.so with gcc if it is not there yet
    return oracle

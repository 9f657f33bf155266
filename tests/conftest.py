import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running test")


def pytest_collection_modifyitems(config, items):
    # GPU tests fail loudly (not skip) when the device or the library is missing:
    # they are only selected with -m gpu on a GPU machine.
    pass


@pytest.fixture(scope="session")
def root():
    return ROOT

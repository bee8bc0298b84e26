import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU-only check")


@pytest.fixture(scope="session")
def olib():
    from oracle import load_lib
    return load_lib("f32")


@pytest.fixture(scope="session")
def olib64():
    from oracle import load_lib
    return load_lib("f64")

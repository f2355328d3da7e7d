import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for p in (ROOT, os.path.join(ROOT, "tests")):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle

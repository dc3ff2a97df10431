import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size (70B-shape) checks that take tens of seconds")


@pytest.fixture(scope="session", autouse=True)
def _host_libs():
    """The two host-side C libraries the tests use: build them only if nothing is built."""
    import synth
    import oracle
    if not os.path.exists(synth.synth._LIB_PATH):
        synth.build()
    if not os.path.exists(oracle.oracle._LIB_PATH):
        oracle.build()
    yield

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    """Build the CPU oracle once per session (plain gcc, a few seconds)."""
    from oracle import build as oracle_build
    if not os.path.exists(oracle_build.LIB):
        oracle_build.build()
    yield


@pytest.fixture(autouse=True)
def _guard_bands(request):
    """Every output the binding allocates in a GPU test is guard-banded and
    the guards are checked after the test (tests/parity.py)."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import parity
    with parity.guard_bands():
        yield

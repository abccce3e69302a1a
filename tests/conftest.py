import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity case (minutes of host work)")


@pytest.fixture(scope="session", autouse=True)
def _host_libraries_built():
    """The oracle and the input generator are small host C libraries; build
    them if a fresh checkout lacks them (the HIP library is built by
    __graft_entry__.build() and is never built from a test)."""
    import __graft_entry__ as ge

    ge.build_host_libraries(only_missing=True)
    yield

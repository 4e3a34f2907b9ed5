import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
for _p in (ROOT, TESTS):
    if _p not in sys.path:
        sys.path.insert(0, _p)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")
    config.addinivalue_line(
        "markers", "slow: full-size workload, tens of GB of device memory")
    config.addinivalue_line("markers", "cpu: runs on the host only")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def pytest_sessionstart(session):
    # Tests load the built library; build it only when none is present.
    import __graft_entry__
    __graft_entry__._build_module().ensure_built()

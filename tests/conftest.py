import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads")


@pytest.fixture(scope="session")
def root_dir():
    return ROOT


def pytest_sessionfinish(session, exitstatus):
    """With PKV_PARITY_RECORD=<file>, write every parity comparison's achieved errors."""
    path = os.environ.get("PKV_PARITY_RECORD")
    if not path:
        return
    from tests import parity
    if not parity.RECORDS:
        return
    with open(path, "w") as f:
        f.write(parity.records_table())

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads")
    # tests/test_host_sanitizers.py runs the host-code tests against a sanitized build of
    # the host C++ with launcher stubs; the binding then loads that library instead
    lib = os.environ.get("PKV_TEST_LIBRARY")
    if lib:
        from paged_kv_cache_26_amd import pkv
        pkv.load_library(lib)


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

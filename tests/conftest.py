import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running statistical test")


def _ensure_host_libs():
    """Build the host-side helper libraries if they are missing (seconds)."""
    import workloads
    import oracle
    if not os.path.exists(workloads.LIB_PATH):
        workloads.build()
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()


_ensure_host_libs()


@pytest.fixture(scope="session")
def nthreads():
    return max(1, min(16, os.cpu_count() or 1))

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running statistical test")


def _stale(lib, src):
    return not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(src)


def _ensure_host_libs():
    """Build the host-side helper libraries if they are missing or older than
    their source (seconds)."""
    import workloads
    import oracle
    if _stale(workloads.LIB_PATH, os.path.join(ROOT, "workloads", "gen.cpp")):
        workloads.build()
    if _stale(oracle.LIB_PATH, os.path.join(ROOT, "oracle", "oracle.cpp")):
        oracle.build()


_ensure_host_libs()


@pytest.fixture(scope="session")
def nthreads():
    return max(1, min(16, os.cpu_count() or 1))

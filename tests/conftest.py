import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionfinish(session, exitstatus):
    try:
        from tests import gpu_util
        gpu_util.flush_records()
    except Exception:  # noqa: BLE001
        pass


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _name_gpu_case(request):
    """Print the case name before a GPU test starts, so a crash names it."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.stderr.write(f"\n[gpu case] {request.node.nodeid}\n")
        sys.stderr.flush()
    yield

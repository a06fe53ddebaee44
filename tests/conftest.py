import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU case on stderr before it runs, so a run that dies
    mid-test still tells which case was on the device."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield

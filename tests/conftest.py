import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size configuration")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    # name each GPU case before it runs, so a fault can be attributed
    if request.node.get_closest_marker("gpu") is not None:
        print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield

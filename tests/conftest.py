import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP path through the C ABI)")
    config.addinivalue_line("markers", "slow: full-size workloads")


@pytest.fixture(autouse=True)
def _announce(request):
    # Name the case before it runs, so a run that dies on the GPU still says which one it was.
    if request.node.get_closest_marker("gpu"):
        print(f"\n[case] {request.node.nodeid}", flush=True)
    yield

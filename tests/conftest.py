import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU cases")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name every GPU case on the real stderr before it runs, so that a run
    that dies on the GPU still says which case it was in."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.__stderr__.write(f"[gpu case] {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield

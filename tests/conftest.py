import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def gpu_available() -> bool:
    import torch
    return torch.cuda.is_available()


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    return oracle


@pytest.fixture(autouse=True)
def _announce_gpu_test(request):
    """Names each GPU test on stderr (flushed) before it touches the device,
    so a run that ends abruptly still shows which case was running."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.stderr.write(f"\n[gpu-test] {request.node.nodeid}\n")
        sys.stderr.flush()
    yield

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")
    config.addinivalue_line("markers", "cpu: runs on the CPU only (no device needed)")


def gpu_available() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def require_gpu():
    if not gpu_available():
        pytest.skip("no GPU visible")


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU case on stderr before it runs, so a run that dies inside a
    kernel still says which case it was."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.stderr.write(f"\n[gpu-case] {request.node.nodeid}\n")
        sys.stderr.flush()
    yield

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds")


@pytest.fixture(scope="session")
def gpu():
    """Skip unless a ROCm device is present; return the library binding."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_exact_attention_amd as rea
    return rea


@pytest.fixture(autouse=True)
def _announce_gpu_test(request):
    """Name each GPU test on the real stderr before it runs (survives a lost box)."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.__stderr__.write(f"[gpu-test] start {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield

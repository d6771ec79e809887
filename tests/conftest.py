import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(autouse=True)
def _gpu_guard(request):
    """A gpu-marked test on a machine without a ROCm device fails loudly
    instead of passing on some fallback."""
    if request.node.get_closest_marker("gpu") is not None:
        import torch
        if not torch.cuda.is_available():
            pytest.fail("this test needs a ROCm GPU (run with -m 'not gpu' on CPU)")
    yield

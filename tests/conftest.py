import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; run with -m gpu")
    config.addinivalue_line("markers", "slow: full-size workloads")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    """The CPU oracle is compiled from source on first use (gcc, a second or so)."""
    from oracle import build
    build.build(force=False)


@pytest.fixture(autouse=True)
def _gpu_required(request):
    """GPU tests fail loudly (never skip) when no GPU is present."""
    if request.node.get_closest_marker("gpu") is not None:
        import torch
        if not torch.cuda.is_available():
            pytest.fail("GPU test run without a GPU")

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a real MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The built C-ABI library, loaded for GPU tests (fails loudly if absent)."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a host without a GPU")
    from post_processing_amd import ws
    return ws.load()

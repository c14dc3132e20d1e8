import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library on cuda:0; the test fails loudly if it is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected but no GPU is visible")
    from chunkwise_kimi_delta_amd import kda
    kda.load()
    return kda

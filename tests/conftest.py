import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def gpu_lib():
    """The built C-ABI library on a visible GPU; fails loudly if either is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a host without a GPU")
    from streaming_causal_video_amd import binding

    return binding.load()

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu():
    """The GPU test context: torch on cuda:0 plus the loaded HIP library.

    Fails (never skips) when no GPU is visible, so a GPU run cannot pass silently
    without executing the kernels.
    """
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import selective_state_space_34_amd as ss
    ss.load()
    return ss

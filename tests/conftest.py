import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes of oracle time)")


@pytest.fixture(scope="session")
def dsa():
    """The HIP library binding; fails loudly when the extension or GPU is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected without a GPU")
    import sparse_attention_long_08_amd as m
    m.load()
    return m

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library binding; GPU tests fail (not skip) when it cannot load."""
    import torch
    assert torch.cuda.is_available(), "gpu tests need a GPU"
    from combine_dispatch_layout_amd import moedl
    moedl.load()
    return moedl


@pytest.fixture(scope="session")
def built_lib():
    """The HIP library loaded without touching a GPU: for host-side argument checks."""
    from combine_dispatch_layout_amd import moedl
    moedl.load()
    return moedl

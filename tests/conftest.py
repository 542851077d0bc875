import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def libqsa():
    """The C-ABI library; built in-tree only if nothing is built yet."""
    from block_sparse_attention_32_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from block_sparse_attention_32_amd import build
        build.build()
    return binding.lib()


@pytest.fixture(scope="session")
def gpu(libqsa):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")

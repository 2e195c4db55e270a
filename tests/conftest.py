import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def gpu():
    """The device for GPU tests.  A gpu-marked test without a device fails instead of skipping, so a
    silent CPU pass cannot hide a missing GPU or library."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("this test needs the GPU; run it with -m gpu on an MI355X")
    from token_sparse_attention_amd import binding
    binding.lib()  # loads libtsa.so or raises
    return torch.device("cuda:0")

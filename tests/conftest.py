import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: runs HIP kernels on an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def gpu():
    """The HIP binding, loaded on a GPU machine; skips where there is no GPU."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from sparse_attention_decode_qsa_amd import binding
    binding.load()
    return binding

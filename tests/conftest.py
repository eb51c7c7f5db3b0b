import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running test")


def _gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    """The loaded native library on a machine with a GPU; skips only where no GPU exists.

    On a machine with a GPU a missing or unloadable library is an error, not
    a skip: the GPU tests must run the HIP path.
    """
    if not _gpu_available():
        pytest.skip("no GPU visible")
    from transformer_attention_06_amd import native
    return native.lib()

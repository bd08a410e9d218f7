import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (long input generation)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library on a GPU.  Skips where no GPU is visible; on a GPU,
    a missing or unloadable library is an error, never a fallback."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import rank_key_sparse_amd as rks
    rks.load_library()  # raises if the built library is missing
    return rks

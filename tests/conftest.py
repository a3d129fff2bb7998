import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library and a GPU, or a loud failure when the GPU is there but
    the library is not."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import io_aware_exact_20_amd as fa
    fa.load()  # raises if the extension is missing
    return fa

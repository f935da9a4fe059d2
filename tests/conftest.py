import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library, loaded, on a machine with a GPU.  GPU tests fail (they
    are not skipped) when the library is missing: a silent fallback would make
    them meaningless."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a GPU")
    import scaled_dot_product_amd as sdpa
    sdpa.library()  # raises when libattn.so is missing or fails to load
    return sdpa

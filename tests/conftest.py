import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large host-memory or long-running CPU case")


@pytest.fixture(scope="session")
def gpu_lib():
    """The built HIP library, loaded once; skips when no GPU is visible."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import fp8_paged_mqa_block_amd as pm

    pm.load_library()  # raises if the library is missing: no fallback exists
    return pm

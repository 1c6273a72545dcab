import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def gpu_available() -> bool:
    import torch
    return torch.cuda.is_available()


@pytest.fixture(scope="session")
def gpu():
    """Skip when no GPU is visible; on a GPU machine the HIP library must load."""
    if not gpu_available():
        pytest.skip("no GPU visible")
    import exact_attention_104_amd as fa
    fa.load_library()  # raises if the HIP extension is missing
    return fa

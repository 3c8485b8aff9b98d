import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


def pytest_collection_modifyitems(config, items):
    # GPU tests run after the CPU ones so that a CPU failure is reported first.
    items.sort(key=lambda it: 1 if it.get_closest_marker("gpu") else 0)


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library bound through ctypes; GPU tests fail loudly if it is absent."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import rmsnorm_nvfp4_block_amd as q

    q.load()  # raises if the shared library is missing
    return q

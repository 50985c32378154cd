import os
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if REPO not in sys.path:
    sys.path.insert(0, REPO)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and libbfq.so")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def orc():
    """The CPU oracle (built with gcc on first use)."""
    import oracle
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    return oracle


@pytest.fixture(scope="session")
def bfq():
    """The ctypes binding of libbfq.so (built with hipcc if it is missing)."""
    from block_scaled_w8a8_amd import build
    if not os.path.exists(build.LIB_PATH):
        build.build()
    from block_scaled_w8a8_amd import bfq as b
    return b


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("a GPU test ran on a machine without a GPU")
    return torch.device("cuda:0")

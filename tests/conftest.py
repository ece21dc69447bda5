import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size workloads")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    return oracle.load()


@pytest.fixture(scope="session")
def gpu():
    """Skips unless a GPU is visible; the HIP library must then load (no fallback)."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import chunkwise_gated_deltanet_amd as cg
    cg.load_library()
    return torch.device("cuda:0")

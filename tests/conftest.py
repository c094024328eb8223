import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (seconds to minutes)")


@pytest.fixture(scope="session")
def gpu():
    """Skip unless a GPU is visible; fail loudly if one is visible but the library is not built."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import mla_kv_cache_amd as m
    m.load()          # raises if the HIP library is missing: no fallback exists
    return torch.device("cuda:0")

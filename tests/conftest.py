import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU work")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def lib():
    """The HIP library binding; GPU tests fail loudly when it is missing."""
    import gram_embedding_layer_amd as g
    return g.load()


@pytest.fixture(scope="session")
def tables_30b():
    """Device tables of the 30B-parameter layer (about 61 GB), shared by the prefill and
    decode tests of that layer."""
    import workloads as WL
    return WL.device_tables(WL.workload("prefill_64k_30b"))

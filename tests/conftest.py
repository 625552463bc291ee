import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(autouse=True)
def _announce_case(request):
    """Names each GPU case on the real stderr before it runs (survives a crash of the process)."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.__stderr__.write(f"CASE {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield


@pytest.fixture(scope="session")
def cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    from int4_blockwise_gemv_amd import vv
    vv.lib()  # fails loudly if the HIP library is missing
    return torch.device("cuda:0")

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(autouse=True)
def _no_expired_waits(request):
    """After every GPU test: no bounded in-kernel wait of the library ran out
    of polls during it (gdn_wait_timeouts reads and clears the device word)."""
    yield
    if request.node.get_closest_marker("gpu") is None:
        return
    import torch
    if not torch.cuda.is_available():
        return
    import gated_deltanet_state_delta_amd as gdn
    assert gdn.wait_timeouts(clear=True) == 0, "an in-kernel wait ran out of polls"

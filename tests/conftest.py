import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(autouse=True)
def _poison_gpu_outputs(request):
    """GPU tests: every output and workspace the binding allocates starts as a
    sentinel (NaN, -2^31, 0xff bytes), so an element a kernel never writes
    cannot carry an earlier call's value into a comparison."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import token_scoring_top_amd as hk
    hk.set_output_poison(True)
    yield
    hk.set_output_poison(False)

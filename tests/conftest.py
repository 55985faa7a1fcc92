import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "debug_flags: feeds malformed routing on purpose")


@pytest.fixture(autouse=True)
def _device_index_checks(request):
    """With a MOE_DEBUG build of the library loaded (MOE_Q4_LIB), every GPU test must leave the
    device index checks clean; tests that feed malformed routing on purpose are marked
    `debug_flags` and check the record themselves."""
    yield
    if request.node.get_closest_marker("gpu") is None or request.node.get_closest_marker("debug_flags"):
        return
    import bit_quantized_expert_top_amd as moe
    flags = moe.moe_debug_status(clear=True)
    assert flags in (None, 0), f"device index checks recorded {flags:#x}"

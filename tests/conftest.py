import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


# A host-only build of the planner (the sanitizer test builds one) can stand
# in for libfia.so: FIA_HOSTCHECK_LIB names it.
if os.environ.get("FIA_HOSTCHECK_LIB"):
    from attention_online_softmax_flash_amd import fia as _fia

    _fia.LIB_PATH = os.environ["FIA_HOSTCHECK_LIB"]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU case on stderr before it touches the device, so a run
    that dies mid-test still says which case was running."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.__stderr__.write(f"\n[gpu case] {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(ROOT)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from tests import hang_guard  # noqa: E402

# Host-side limits of the GPU hang guard (tests/hang_guard.py), in seconds:
# the whole test body, then the drain of the work it left on its stream.
HANG_BODY_LIMIT_S = float(os.environ.get("SPA_HANG_GUARD_S", "100"))
HANG_DRAIN_LIMIT_S = 20.0


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: larger CPU cases")


@pytest.fixture(autouse=True)
def gpu_hang_guard(request):
    """Every GPU test runs under a watchdog and ends with a bounded drain of
    its stream; either limit ends the process with the test's id."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    nodeid = request.node.nodeid
    dog = hang_guard.Watchdog(
        HANG_BODY_LIMIT_S,
        lambda: hang_guard.report_and_exit(nodeid, "the test body", HANG_BODY_LIMIT_S))
    try:
        yield
        import torch
        if torch.cuda.is_available():
            stream = torch.cuda.current_stream()
            hang_guard.drain(
                stream.query, HANG_DRAIN_LIMIT_S,
                lambda: hang_guard.report_and_exit(nodeid, "the work left on its stream",
                                                   HANG_DRAIN_LIMIT_S))
    finally:
        dog.stop()

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="module")
def side_stream_always():
    """Run the ring's staging copies on the side stream at every size. The
    library runs the copies of blocks under 32 MiB in order on the compute
    stream; the small GPU tests use this fixture so that they exercise the
    two-stream path (events, double buffer), which the full-size workloads
    take by default."""
    old = os.environ.get("RA_SIDE_STREAM_MIN_BYTES")
    os.environ["RA_SIDE_STREAM_MIN_BYTES"] = "0"
    yield
    if old is None:
        os.environ.pop("RA_SIDE_STREAM_MIN_BYTES", None)
    else:
        os.environ["RA_SIDE_STREAM_MIN_BYTES"] = old

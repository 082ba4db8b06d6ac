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


@pytest.fixture(scope="module", params=["8", "4"])
def both_forward_shapes(request):
    """Run the module once with 8-wave and once with 4-wave workgroups of the
    bf16 attention kernel. The library picks 4 waves only for shares whose
    8-wave grid has fewer workgroups than the GPU has CUs, which is every
    small test here; forcing each keeps both kernels under every case."""
    old = os.environ.get("RA_WAVES")
    os.environ["RA_WAVES"] = request.param
    yield request.param
    if old is None:
        os.environ.pop("RA_WAVES", None)
    else:
        os.environ["RA_WAVES"] = old

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # a GPU test asked for on a machine without one is an error, not a skip
    pass


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.lib()
    return oracle


@pytest.fixture(autouse=True)
def _announce_gpu_test(request):
    """Name each GPU test on stderr before it runs, so a run that dies on the
    device still says which case it was in."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.stderr.write(f"\n[gpu-test] {request.node.nodeid}\n")
        sys.stderr.flush()
    yield

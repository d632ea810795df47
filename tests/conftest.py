import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    # The oracle is test infrastructure; build it if this checkout has no copy.
    from oracle.build import LIB, build_oracle

    if not os.path.exists(LIB):
        build_oracle()
    yield


def pytest_runtest_logstart(nodeid, location):
    # Name the case on the raw stderr before it runs, so a run that dies on
    # the GPU still says which test it was in.
    if "gpu" in nodeid or "parity" in nodeid or "determinism" in nodeid:
        sys.__stderr__.write("[start] %s\n" % nodeid)
        sys.__stderr__.flush()

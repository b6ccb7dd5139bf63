import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libpa.so")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    """The oracle is C; build it once per session if it is missing."""
    import oracle
    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        oracle.build()
    yield


@pytest.fixture
def report(request):
    """print() that reaches the terminal even while pytest captures output:
    for figures a test is asked to report (error statistics, the fp8
    quantisation effect)."""
    capman = request.config.pluginmanager.getplugin("capturemanager")

    def _report(msg: str) -> None:
        with capman.global_and_fixture_disabled():
            print(msg, flush=True)
    return _report

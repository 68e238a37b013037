import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)

import parity_report  # noqa: E402


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(autouse=True)
def _parity_test_name(request):
    parity_report.CURRENT[0] = request.node.nodeid
    yield


def pytest_sessionfinish(session, exitstatus):
    path = parity_report.write(ROOT, "2e-3 + 1e-2 |ref|", "1e-4 + 1e-3 |ref|")
    if path:
        print(f"\nparity exception counts written to {path}", flush=True)

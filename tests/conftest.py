import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case (minutes)")


@pytest.fixture(scope="session")
def olib():
    import oracle
    return oracle.lib()


def pytest_terminal_summary(terminalreporter):
    """Per-case parity counts (exact ties, near-tie tokens) collected by the
    GPU tests; printed even under -q."""
    try:
        from tests import harness
    except Exception:
        return
    if harness.REPORT:
        terminalreporter.section("parity summary")
        for line in harness.REPORT:
            terminalreporter.write_line(line)

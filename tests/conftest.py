import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.default()


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Worst GPU-vs-oracle errors per case family and dtype (GPU runs only)."""
    mod = sys.modules.get("gpu_util")
    if mod is None or not getattr(mod, "RECORD", None):
        return
    terminalreporter.write_sep("=", "parity: worst |gpu - oracle| per case family and dtype")
    for line in mod.summary_lines():
        terminalreporter.write_line(line)

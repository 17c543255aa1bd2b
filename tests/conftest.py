import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def O():
    """The CPU oracle (test infrastructure)."""
    from oracle import oracle
    oracle.lib()
    return oracle


def pytest_terminal_summary(terminalreporter):
    """The measured parity margins of the block-scaled GEMM checks (worst |D - ref| / sum|ab|
    per case, against the stated bound of 1e-5), printed even when every test passes."""
    mod = sys.modules.get("mx_check")
    if mod is None or not mod.MARGINS:
        return
    terminalreporter.write_sep("-", "block-scaled parity margins: worst |D-ref|/sum|ab| (bound 1e-5)")
    for name, worst in sorted(mod.MARGINS.items()):
        terminalreporter.write_line(f"{name}: {worst:.3e}")

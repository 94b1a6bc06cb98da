import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # build the CPU oracle only when nothing is built yet
    lib = os.path.join(ROOT, "oracle", "liboracle.so")
    if not os.path.exists(lib):
        from oracle.build import build
        build()


@pytest.fixture(scope="session")
def repo_root():
    return ROOT


def pytest_terminal_summary(terminalreporter):
    """The largest relative error each dtype reached against the oracle in this run."""
    par = sys.modules.get("_parity")  # imported by the GPU parity tests only
    if par is None:
        return
    TOL, WORST = par.TOL, par.WORST
    for dt, (rel, what) in sorted(WORST.items(), key=lambda kv: str(kv[0])):
        terminalreporter.write_line(f"parity margin {dt}: worst max|err|/max|ref| {rel:.3e} ({what}) "
                                    f"vs tolerance {TOL[dt]:.0e}")

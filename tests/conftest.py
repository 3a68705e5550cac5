import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """The session's parity margins (tests/margins.py), also under -q; with
    DFLASH_MARGINS set, the full list is written to that file too."""
    import margins

    for line in margins.summary_lines():
        terminalreporter.write_line(line)
    path = os.environ.get("DFLASH_MARGINS")
    if path and margins.RECORDS:
        with open(path, "w") as f:
            for what, err, tol in margins.RECORDS:
                f.write(f"{err / tol if tol else float('inf'):.6f}\t{err:.4e}\t{tol:.4e}\t{what}\n")


@pytest.fixture(scope="session")
def orc():
    from oracle import oracle as O
    O.build()
    return O

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


def pytest_terminal_summary(terminalreporter):
    parity = sys.modules.get("parity")
    if parity is not None and sum(parity.REF_STATS.values()):
        terminalreporter.write_line(f"oracle references: {parity.REF_STATS['stored']} stored, "
                                    f"{parity.REF_STATS['computed']} computed on the spot")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle

    alt = os.environ.get("ORACLE_LIB")   # set by the mutation and sanitizer tests, which run other builds
    if alt:
        oracle.use_library(alt)
    else:
        oracle.build(force=False)
    return oracle

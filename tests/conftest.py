import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: larger CPU case")


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.get()


@pytest.fixture(autouse=True, scope="session")
def _carry_checks():
    """Every scan and backward call of the GPU tests checks its workspace's
    carry error word afterwards (a timed-out carry wait fails the test)."""
    import selective_state_space_80_amd as mamba
    mamba.set_carry_checks(True)
    yield
    mamba.set_carry_checks(False)

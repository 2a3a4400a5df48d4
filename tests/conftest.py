import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size workload parity (minutes of oracle time)")


@pytest.fixture(scope="session", autouse=True)
def _built_host_libs():
    """The oracle and the input generator are plain C; build them once."""
    import oracle
    import synth
    oracle.build()
    synth.build()

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session", autouse=True)
def _built_libraries():
    """Build whatever is missing (gcc for the oracle and the generator, hipcc
    for the GPU library); an existing build is used as it is."""
    import __graft_entry__ as g

    g.ensure_built()

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, TESTS):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _ensure_built(path):
    """Build only when nothing is built yet (the build step is __graft_entry__.build())."""
    if not os.path.exists(path):
        import __graft_entry__
        __graft_entry__.build()


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    _ensure_built(oracle.DEFAULT_LIB)
    return oracle.default()

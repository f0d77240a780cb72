import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size layer cases (minutes on the CPU oracle)")


@pytest.fixture(scope="session")
def slib():
    """The C-ABI library, (re)built first if a source is newer than it."""
    from free_activation_sparse_amd import build as _build
    import free_activation_sparse_amd as fas
    if _build.is_stale():
        _build.build()
    return fas

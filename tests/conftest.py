import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.lib()  # builds the C oracle if it is missing or stale
    return oracle


@pytest.fixture(scope="session")
def native():
    """The HIP library's ctypes binding. Builds it first only if nothing is
    built (a fresh checkout); otherwise loads what is there."""
    import sparse_attention_decode_row_amd as pkg
    if not os.path.exists(pkg.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    return pkg

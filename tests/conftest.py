import os
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a gfx950 GPU (run through the HIP library)")


@pytest.fixture(scope="session")
def jetlib():
    """The C-ABI library, built in-tree if it is not there yet."""
    from quantized_rl_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from quantized_rl_amd import build
        build.build()
    return _lib.lib()

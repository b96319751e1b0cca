import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size oracle work (tens of seconds)")


@pytest.fixture(scope="session")
def lib():
    """The loaded C-ABI library (skips when it has not been built)."""
    from weight_only_bit_group_amd import _lib
    try:
        return _lib.load()
    except OSError as exc:  # pragma: no cover - depends on the build
        pytest.skip(f"libaq.so not built: {exc}")

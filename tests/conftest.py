import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; parity against the oracle")


@pytest.fixture(autouse=True)
def _dispatch_config_restored():
    """Tests that set W4_* dispatch variables (monkeypatch, undone before this
    fixture's teardown) leave the library's configuration as the environment
    is after them."""
    yield
    import bit_weight_only_w4a16_amd as w4
    if w4._lib is not None:
        w4.config_reload()


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.build()
    return oracle

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# The library reads its tuning overrides (QR_GEMV_*, QR_GEMM_*, ...) and QR_TRACE only when QR_TUNE is set at
# load time; the tests force kernel variants through them, so the switch is set before anything loads libqr.so.
os.environ.setdefault("QR_TUNE", "1")
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libqr.so")
    config.addinivalue_line("markers", "slow: long CPU test (exhaustive sweeps); run with -m slow")


def pytest_collection_modifyitems(config, items):
    # exhaustive CPU sweeps run only when asked for by marker expression
    expr = config.getoption("-m") or ""
    if "slow" in expr:
        return
    skip = pytest.mark.skip(reason="slow exhaustive sweep: select with -m slow")
    for item in items:
        if "slow" in item.keywords:
            item.add_marker(skip)

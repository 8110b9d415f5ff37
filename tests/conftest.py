import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


_CAPTURE = None


def pytest_configure(config):
    global _CAPTURE
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    _CAPTURE = config.pluginmanager.getplugin("capturemanager")


def progress(msg):
    """Print msg at once, past pytest's output capture, so that a long test (the full-size
    layers spend minutes in the float64 oracle) shows its steps while it runs."""
    if _CAPTURE is None:
        print(msg, flush=True)
        return
    with _CAPTURE.global_and_fixture_disabled():
        print(msg, flush=True)


@pytest.fixture(scope="session")
def golden_dir():
    return GOLDEN

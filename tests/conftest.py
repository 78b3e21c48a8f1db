import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture
def tuning_library():
    """Route the binding through libfbob_tuning.so (the measurement build, in which
    FBOB_TUNE_* variables select kernel variants) for the duration of a test."""
    from exact_softmax_attention_fbob_amd import _lib
    with _lib.using_library(_lib.tuning_library_path()):
        yield

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(autouse=True)
def _default_dtype_unchanged():
    """No test may leave torch's default dtype changed for the ones after it."""
    import torch
    before = torch.get_default_dtype()
    yield
    assert torch.get_default_dtype() == before, "a test changed torch's default dtype"

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built libbitlinear")


@pytest.fixture(scope="session")
def gpu():
    """The GPU binding, on a machine with a GPU.  No GPU -> skip; a GPU but no
    built library -> the binding's own import error, loudly."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this machine")
    import ternary_weight_linear_absmean_amd as bl
    bl.load()          # raises if libbitlinear.so is missing or fails to load
    return bl

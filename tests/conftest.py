import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def fd():
    """The HIP-backed Python binding; GPU tests only."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("gpu-marked test run without a visible GPU")
    import decode_attention_06_amd as fdmod

    fdmod.load()          # raises if the shared library is missing
    return fdmod

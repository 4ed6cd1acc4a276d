import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU work of more than a few seconds")


@pytest.fixture(scope="session")
def lib():
    """The C-ABI library through its Python binding (no device needed to load it)."""
    from invariant_lm_head_deterministic_amd import _lib

    return _lib.load()


@pytest.fixture(scope="session")
def rlk():
    """The binding module with a GPU present; fails loudly when the HIP library is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import invariant_lm_head_deterministic_amd as rlk

    rlk.require_library()
    return rlk

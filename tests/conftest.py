import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its Python binding; only for tests marked gpu."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from context_mla_prefill_amd import _lib
    _lib.load()  # raises if the built library is missing
    return _lib

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    """The HIP library bound to cuda:0; a GPU test fails loudly without it."""
    if not _gpu_available():
        pytest.fail("GPU test run without a visible GPU")
    from paged_kv_decode_attention_amd import ops
    ops.load_library()  # raises if the shared library is missing
    return ops

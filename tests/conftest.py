import os
import sys

import pytest

try:  # import torch once at collection: the first import on a fresh box is slow
    import torch  # noqa: F401
except Exception:  # pragma: no cover
    torch = None

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU-side work (full-size oracle runs)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library on a real GPU; fails loudly when either is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a host without a GPU (run with -m 'not gpu')")
    import unstructured_sparse_transformer_amd as twell
    twell.load()  # raises if libtwell.so was not built
    return twell

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu():
    """The HIP library bound to cuda:0; fails loudly when the GPU or the library is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("a gpu-marked test ran without a visible GPU")
    import dense_tiled_gemm_amd as gb

    gb.load()  # raises if the shared library is not built
    return gb

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle

    return oracle.load()


@pytest.fixture(scope="session")
def pa():
    """The HIP library binding; fails loudly when the library or the GPU is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test collected without a GPU: run with -m 'not gpu' on CPU hosts")
    import paged_attention_quantized_amd as pa_mod

    pa_mod.load()
    return pa_mod

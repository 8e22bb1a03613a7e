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
    """The built HIP library through its Python binding, on cuda:0."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("a gpu-marked test ran without a visible GPU")
    from exact_head_attention_amd import binding
    return binding

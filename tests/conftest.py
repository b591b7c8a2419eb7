"""Shared pytest setup: the ``gpu`` marker, repo import path, and GPU availability."""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP path's Python binding, loaded; GPU tests fail loudly if it is not built."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    import online_softmax_attention_fa_amd as fa

    fa.load()  # raises if libfa.so is missing
    return fa

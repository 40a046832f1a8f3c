"""pytest configuration: the ``gpu`` marker and shared helpers.

Tests marked ``gpu`` need an MI355X and the built HIP library; everything else
runs on the CPU (``-m "not gpu"``).
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library; fails (not skips) when it is missing on a GPU run."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from tiled_attention_05_amd import _lib
    return _lib.load()

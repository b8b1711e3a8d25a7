"""Shared pytest configuration: the ``gpu`` marker and small tensor helpers."""

import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def bits(t):
    """Raw bf16 bit patterns of a torch tensor as numpy.uint16 (on the CPU)."""
    import torch
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def npy(t):
    """A torch tensor as a numpy array on the CPU (no dtype change)."""
    return t.detach().cpu().numpy()


@pytest.fixture
def golden_dir():
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

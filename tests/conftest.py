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


# -------------------------------------------------------------- parity helpers

ATOL = 2e-3   # absolute bound on max |gpu - oracle| for attention outputs
RTOL = 1e-2   # relative bound, normwise: max |gpu - oracle| <= RTOL * max |oracle|


def assert_attention_close(gpu, ref, what="out"):
    """bf16 inputs, fp32 accumulation: (A) max|err| <= 2e-3 and (B) max|err| <= 1e-2 max|ref|,
    which also implies the elementwise allclose(atol=2e-3, rtol=1e-2)."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    finite = np.isfinite(r)
    assert np.array_equal(finite, np.isfinite(g)), f"{what}: non-finite pattern differs"
    if not finite.any():
        return
    err = np.abs(g[finite] - r[finite])
    scale = np.max(np.abs(r[finite]))
    assert err.max() <= ATOL, f"{what}: max abs err {err.max():.3e} > {ATOL}"
    assert err.max() <= RTOL * max(scale, 1e-30), f"{what}: max err {err.max():.3e} > {RTOL} * {scale:.3e}"
    assert np.allclose(g, r, atol=ATOL, rtol=RTOL, equal_nan=True)


def assert_lse_close(gpu, ref):
    """lse = log-sum-exp of the scaled scores (natural log); -inf where nothing is attended."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert np.array_equal(np.isneginf(g), np.isneginf(r))
    m = np.isfinite(r)
    if m.any():
        assert np.max(np.abs(g[m] - r[m])) <= ATOL * max(1.0, np.max(np.abs(r[m])))

"""Shared test set-up: the `gpu` marker, device fixtures, byte comparison.

GPU tests call the HIP library through its C ABI (via the ctypes binding) on
cuda:0; CPU tests cover the oracle, the host logic and the library's symbol
table. Nothing here reads anything outside the repository.
"""

from __future__ import annotations

import hashlib
import os
import sys
from pathlib import Path

import numpy as np
import pytest

REPO = Path(__file__).resolve().parent.parent
if str(REPO) not in sys.path:
    sys.path.insert(0, str(REPO))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP kernels)")
    config.addinivalue_line("markers", "slow: long CPU test")


def _gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(scope="session")
def built_library():
    """Path of the shared library; builds the libraries once if one is
    missing or was built from other sources than the tree's."""
    from hyper_connection_residual_mhc_amd import _build
    _build.ensure_built()
    return _build.LIB_PATH


@pytest.fixture(scope="session")
def device(built_library):
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    return dev


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def assert_bytes_equal(got: np.ndarray, want: np.ndarray, what: str) -> None:
    """Raw-bit equality with the first differing flat index in the message
    (-0 and +0 differ, NaN patterns compare by bits)."""
    got = np.ascontiguousarray(got)
    want = np.ascontiguousarray(want)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    assert got.dtype.itemsize == want.dtype.itemsize
    g = got.view(f"u{got.dtype.itemsize}").ravel()
    w = want.view(f"u{want.dtype.itemsize}").ravel()
    if not np.array_equal(g, w):
        bad = np.flatnonzero(g != w)
        i = int(bad[0])
        idx = np.unravel_index(i, got.shape)
        raise AssertionError(
            f"{what}: {bad.size} of {g.size} differ; first at {idx}: "
            f"got 0x{int(g[i]):x}, want 0x{int(w[i]):x}; "
            f"sha256 got {digest(got)[:16]} want {digest(want)[:16]}")

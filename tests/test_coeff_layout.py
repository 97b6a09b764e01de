"""The coefficient epilogue's kernels follow the oracle's row order.

The kernels lay the fixed two-stage order out on hardware as follows:

* chunk stage: wave c owns rows 64c .. 64c+63, lane r one row; each lane
  writes its m + 3 summed values into an LDS tile, value-major with a row
  stride of 68 floats (n = 8's 83 values in passes of at most 64), then lane
  v reads value v's 64 entries and runs the halving tree on them in its own
  registers; the chunk sum of value v goes to partial[v * chunks + c];
* second stage, one-launch form: the last block's W waves (W = 2 up to 64
  chunks, 4 above) split the m + 3 outputs, Q = ceil((m + 3) / W) per wave,
  output v = w * Q + q; lane l adds partial[v * chunks + 64k + l] for
  k = 0, 1, ... in ascending order (past the last chunk: +0.0), then the
  halving tree across the wave;
* second stage, two-launch form: one wave per output, the same walk.

These CPU tests emulate those index maps with explicit loops (numpy float32,
one rounding per addition) and compare the bits with oracle.coeff_bwd, so a
wrong stride, offset or output split shows up without a GPU.
"""

from __future__ import annotations

import numpy as np
import pytest

from oracle import coeff_bwd as CB

F = np.float32
STRIDE = 68


def _tree(x: np.ndarray) -> np.float32:
    x = x.copy()
    off = 32
    while off >= 1:
        for j in range(off):
            x[j] = F(x[j] + x[j + off])
        off //= 2
    return x[0]


def chunk_stage(vals: np.ndarray) -> np.ndarray:
    """vals [R, V] (the per-row summed values) -> partial [V * chunks] in
    the kernels' layout, through the LDS tile."""
    R, V = vals.shape
    chunks = -(-R // 64)
    partial = np.full(V * chunks, np.nan, np.float32)
    for c in range(chunks):
        rows = np.zeros((64, V), np.float32)
        valid = min(64, R - 64 * c)
        rows[:valid] = vals[64 * c:64 * c + valid]
        for base in range(0, V, 64):
            cnt = min(64, V - base)
            tile = np.full(64 * STRIDE, np.nan, np.float32)
            for lane in range(64):                     # each lane writes its row's values
                for i in range(cnt):
                    tile[i * STRIDE + lane] = rows[lane, base + i]
            for lane in range(cnt):                    # lane v reduces value v
                partial[(base + lane) * chunks + c] = _tree(tile[lane * STRIDE:lane * STRIDE + 64])
    assert not np.isnan(partial).any()
    return partial


def output_walk(partial: np.ndarray, v: int, chunks: int) -> np.float32:
    acc = np.zeros(64, np.float32)
    for k in range(-(-chunks // 64)):
        for lane in range(64):
            idx = 64 * k + lane
            x = partial[v * chunks + idx] if idx < chunks else F(0.0)
            acc[lane] = F(acc[lane] + x)
    return _tree(acc)


def one_launch_outputs(partial: np.ndarray, V: int, chunks: int) -> np.ndarray:
    W = 2 if chunks <= 64 else 4
    Q = -(-V // W)
    out = np.full(V, np.nan, np.float32)
    for w in range(W):
        for q in range(Q):
            v = w * Q + q
            if v < V:
                out[v] = output_walk(partial, v, chunks)
    return out


def _values(R: int, n: int, seed: int) -> np.ndarray:
    """The m + 3 per-row summed values the kernels reduce: d of every column,
    then the three group sums e."""
    rng = np.random.default_rng(seed)
    m = CB.columns(n)
    f = lambda *s: rng.standard_normal(s).astype(np.float32)  # noqa: E731
    pre = rng.random((R, n), dtype=np.float32)
    post = rng.random((R, n), dtype=np.float32) * F(2.0)
    d = CB.dz(pre, post, f(R, n), f(R, n), f(R, n * n), 2.0)
    mix = f(R, m)
    k = CB.groups(n)
    e = np.zeros((R, 3), np.float32)
    for j in range(m):
        e[:, k[j]] = np.add(e[:, k[j]], np.multiply(d[:, j], mix[:, j]))
    return np.concatenate([d, e], axis=1)


@pytest.mark.parametrize("n,R", [(2, 1), (4, 63), (4, 200), (8, 130), (2, 4096), (4, 4097)])
def test_kernel_layouts_give_the_oracle_row_sums(n, R):
    vals = _values(R, n, seed=R + n)
    V = vals.shape[1]
    chunks = -(-R // 64)
    want = CB.row_sum(vals)
    partial = chunk_stage(vals)
    one = one_launch_outputs(partial, V, chunks)
    two = np.array([output_walk(partial, v, chunks) for v in range(V)], np.float32)
    assert np.array_equal(one.view(np.uint32), want.view(np.uint32))
    assert np.array_equal(two.view(np.uint32), want.view(np.uint32))


def test_a_wrong_partial_stride_is_detected():
    """Storing chunk sums chunk-major (partial[c * V + v]) while reading them
    output-major picks up other outputs' sums."""
    R, n = 300, 4
    vals = _values(R, n, seed=5)
    V = vals.shape[1]
    chunks = -(-R // 64)
    good = chunk_stage(vals)
    wrong = good.reshape(V, chunks).T.reshape(-1).copy()
    got = np.array([output_walk(wrong, v, chunks) for v in range(V)], np.float32)
    assert not np.array_equal(got.view(np.uint32), CB.row_sum(vals).view(np.uint32))

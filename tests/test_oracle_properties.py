"""Property checks of the oracles on random inputs (hypothesis, CPU).

Each property holds exactly, bit for bit, for the fixed orders the oracles
define, and fails for plausible mistakes in them:

* the grad_pre order (oracle.h_aggregate.canonical_tree_sum) and the
  coefficient epilogue's row order (oracle.coeff_bwd.row_sum) are odd
  functions (round to nearest is symmetric), commute with scaling by a power
  of two while nothing overflows or underflows, ignore appended zeros (the
  accumulators start at +0.0 and adding +0.0 changes no value), and return a
  lone non-zero term unchanged;
* the forward is odd in the residual and commutes with power-of-two scaling
  of pre in the same way, and is unchanged by swapping the streams inside a
  pair or the two pairs of its (0+1)+(2+3) tree.
"""

from __future__ import annotations

import numpy as np
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

from hyper_connection_residual_mhc_amd.workloads import to_bf16_bits  # noqa: E402
from oracle import coeff_bwd as CB  # noqa: E402
from oracle import h_aggregate as O  # noqa: E402

SETTINGS = settings(max_examples=40, deadline=None, derandomize=True)


def _values(seed: int, shape, spread: float = 8.0) -> np.ndarray:
    """float32 values of either sign whose magnitudes span 2^-spread..2^spread
    (no overflow or underflow under the scalings below)."""
    rng = np.random.default_rng(seed)
    mag = np.exp2(rng.uniform(-spread, spread, shape))
    sign = np.where(rng.random(shape) < 0.5, -1.0, 1.0)
    return (sign * mag).astype(np.float32)


def _same(a, b) -> bool:
    return np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b).view(np.uint32))


@SETTINGS
@given(H=st.integers(1, 2600), seed=st.integers(0, 2**31), k=st.integers(-20, 20),
       pad=st.integers(1, 700))
def test_grad_pre_order_properties(H, seed, k, pad):
    q = _values(seed, (2, H))
    s = O.canonical_tree_sum(q)
    assert _same(O.canonical_tree_sum(-q), -s)
    scale = np.float32(2.0 ** k)
    assert _same(O.canonical_tree_sum(q * scale), s * scale)
    padded = np.concatenate([q, np.zeros((2, pad), np.float32)], axis=1)
    assert _same(O.canonical_tree_sum(padded), s)
    lone = np.zeros((1, H), np.float32)
    h = seed % H
    lone[0, h] = q[0, h]
    assert _same(O.canonical_tree_sum(lone), q[0, h:h + 1])


@SETTINGS
@given(R=st.integers(1, 9000), seed=st.integers(0, 2**31), k=st.integers(-20, 20),
       pad=st.integers(1, 300))
def test_coefficient_row_order_properties(R, seed, k, pad):
    x = _values(seed, (R, 3))
    s = CB.row_sum(x)
    assert _same(CB.row_sum(-x), -s)
    scale = np.float32(2.0 ** k)
    assert _same(CB.row_sum(x * scale), s * scale)
    assert _same(CB.row_sum(np.concatenate([x, np.zeros((pad, 3), np.float32)])), s)
    lone = np.zeros((R, 3), np.float32)
    r = seed % R
    lone[r] = x[r]
    assert _same(CB.row_sum(lone), x[r])


@SETTINGS
@given(T=st.integers(1, 6), H=st.integers(1, 300), seed=st.integers(0, 2**31),
       k=st.integers(-20, 20))
def test_forward_properties(T, H, seed, k):
    rng = np.random.default_rng(seed)
    res = to_bf16_bits(_values(seed, (T, 4, H), spread=6.0))
    pre = rng.random((T, 4), dtype=np.float32) + np.float32(0.5)
    out = O.h_aggregate_fwd(res, pre)
    # odd in the residual: flipping every sign bit flips the result's
    assert np.array_equal(O.h_aggregate_fwd(res ^ np.uint16(0x8000), pre), out ^ np.uint16(0x8000))
    # pre scaled by a power of two scales every product and sum exactly
    scaled = O.h_aggregate_fwd(res, pre * np.float32(2.0 ** k))
    want = O.bf16_rne(O.widen_bf16(out) * np.float32(2.0 ** k))
    assert np.array_equal(scaled, want)
    # the tree's symmetries: swap inside a pair, swap the pairs
    for perm in ((1, 0, 2, 3), (0, 1, 3, 2), (2, 3, 0, 1)):
        assert np.array_equal(O.h_aggregate_fwd(res[:, perm, :].copy(), pre[:, perm].copy()), out)

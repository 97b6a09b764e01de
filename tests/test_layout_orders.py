"""The backward's two thread layouts follow the oracle's summation order.

Each kernel layout arranges the fixed order differently on hardware lanes:

* split layout: the 256 accumulator lanes are a block's 256 threads; thread
  l adds groups l, l+256, ... and the four 64-lane halving trees meet in LDS;
* row layout: one 64-lane wave per row; lane j keeps four accumulators,
  acc[m] standing for accumulator lane j + 64m, visits groups j + 64c in
  ascending c and adds group j + 64c into acc[c mod 4]; the halving tree
  runs on each acc[m] across the wave, and lane 0 combines the four.

These CPU tests emulate each layout step by step (numpy float32, one
rounding per addition, explicit loops in the layout's own indexing) and
compare the bits with the oracle's canonical order. They pin the
re-indexing argument the kernels rely on, independently of any GPU.
"""

from __future__ import annotations

import numpy as np
import pytest

from oracle import h_aggregate as O

F = np.float32


def halving_tree(x: np.ndarray) -> np.float32:
    """64 values, x[j] += x[j + off] for off = 32..1; returns x[0]."""
    x = x.copy()
    off = 32
    while off >= 1:
        for j in range(off):
            x[j] = F(x[j] + x[j + off])
        off //= 2
    return x[0]


def split_layout_sum(q: np.ndarray) -> np.float32:
    H = q.size
    acc = np.zeros(256, F)
    for thread in range(256):
        k = thread
        while 8 * k < H:
            for h in range(8 * k, min(8 * k + 8, H)):
                acc[thread] = F(acc[thread] + q[h])
            k += 256
    y = [halving_tree(acc[64 * w:64 * w + 64]) for w in range(4)]
    return F(F(y[0] + y[2]) + F(y[1] + y[3]))


def row_layout_sum(q: np.ndarray, ring: int = 8) -> np.float32:
    """Lane j of the wave, chunk c (groups j + 64c), processed round by round
    through a ring of `ring` slots as the kernel does (the visiting order of
    one lane's chunks is ascending c either way)."""
    H = q.size
    ngroups = -(-H // 8)
    chunks = -(-ngroups // 64)
    rounds = -(-chunks // ring)
    acc = np.zeros((64, 4), F)                   # [lane j][m]
    for j in range(64):
        for r in range(rounds):
            for b in range(ring):
                c = r * ring + b
                k = j + 64 * c                   # this slot's group
                for h in range(8 * k, min(8 * k + 8, H)):   # zeros past H add nothing
                    acc[j, b % 4] = F(acc[j, b % 4] + q[h])
    y = [halving_tree(acc[:, m]) for m in range(4)]
    return F(F(y[0] + y[2]) + F(y[1] + y[3]))


@pytest.mark.parametrize("H", [1, 7, 8, 9, 511, 513, 2048, 2056, 4100, 7168, 7175])
def test_both_layouts_give_the_oracle_bits(H):
    rng = np.random.default_rng(H)
    # wide magnitudes so that a different association changes the bits
    q = (rng.standard_normal(H) * np.exp2(rng.integers(-12, 12, H))).astype(F)
    want = O.canonical_tree_sum(q[None, :])[0]
    assert split_layout_sum(q).view(np.uint32) == want.view(np.uint32)
    for ring in (4, 8, 12):
        assert row_layout_sum(q, ring).view(np.uint32) == want.view(np.uint32), ring


def test_a_wrong_accumulator_index_is_detected():
    """Self-check of the emulation's power: giving chunk c to acc[c // 4 % 4]
    instead of acc[c % 4] (a plausible indexing slip) changes the bits."""
    H = 7168
    rng = np.random.default_rng(1)
    q = (rng.standard_normal(H) * np.exp2(rng.integers(-12, 12, H))).astype(F)
    want = O.canonical_tree_sum(q[None, :])[0]
    ngroups = H // 8
    acc = np.zeros((64, 4), F)
    for j in range(64):
        for c in range(-(-ngroups // 64)):
            k = j + 64 * c
            for h in range(8 * k, min(8 * k + 8, H)):
                acc[j, (c // 4) % 4] = F(acc[j, (c // 4) % 4] + q[h])
    y = [halving_tree(acc[:, m]) for m in range(4)]
    wrong = F(F(y[0] + y[2]) + F(y[1] + y[3]))
    assert wrong.view(np.uint32) != want.view(np.uint32)

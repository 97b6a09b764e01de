"""The streaming probe (measurement library, beside the operation) moves
exactly the bytes its header describes: per unit, `reads` KiB in and
`writes` KiB out, each written 16-byte vector the XOR of the unit's loaded
vectors at that lane (a write-only unit: its unit index), and nothing
written outside dst."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_util import say
from hyper_connection_residual_mhc_amd import probes

pytestmark = pytest.mark.gpu

KiB = 1024


def expected(src: np.ndarray, reads: int, writes: int) -> np.ndarray:
    """dst words from src words (uint32), written out unit by unit."""
    units = src.size * 4 // (reads * KiB)
    x = src.reshape(units, reads, 64, 4)       # unit, chunk, lane, word
    acc = np.bitwise_xor.reduce(x, axis=1)     # unit, lane, word
    return np.repeat(acc[:, None], writes, axis=1).reshape(-1)


@pytest.mark.parametrize("reads,writes", [(1, 1), (4, 1), (5, 4), (9, 4)])
@pytest.mark.parametrize("units", [1, 3, 257])
def test_stream_probe_moves_the_described_bytes(device, reads, writes, units):
    say(f"stream probe {reads}:{writes} units={units}")
    rng = np.random.default_rng(reads * 100 + writes + units)
    src_words = rng.integers(0, 2**32, size=units * reads * KiB // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(src_words.view(np.int32)).to(device)
    guard = 4096
    buf = torch.full((units * writes * KiB // 4 + 2 * guard,), -1, dtype=torch.int32, device=device)
    dst = buf[guard:guard + units * writes * KiB // 4]
    probes.mhc_stream_probe(src, dst, reads, writes)
    torch.cuda.synchronize()
    got = buf.cpu().numpy().view(np.uint32)
    assert np.array_equal(got[guard:-guard], expected(src_words, reads, writes))
    assert (got[:guard] == 0xFFFFFFFF).all() and (got[-guard:] == 0xFFFFFFFF).all()


@pytest.mark.parametrize("units", [1, 5, 300])
def test_read_only_probe_reads_and_writes_nothing(device, units):
    say(f"stream probe 8:0 units={units}")
    src = torch.arange(units * 8 * KiB // 4, dtype=torch.int32, device=device)
    before = src.clone()
    probes.mhc_stream_probe(src, None, 8, 0)
    torch.cuda.synchronize()
    assert torch.equal(src, before)


@pytest.mark.parametrize("units", [1, 5, 300])
def test_write_only_probe_writes_its_unit_index(device, units):
    say(f"stream probe 0:8 units={units}")
    guard = 4096
    buf = torch.full((units * 8 * KiB // 4 + 2 * guard,), -1, dtype=torch.int32, device=device)
    dst = buf[guard:guard + units * 8 * KiB // 4]
    probes.mhc_stream_probe(None, dst, 0, 8)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    want = np.repeat(np.arange(units, dtype=np.int32), 8 * KiB // 4)
    assert np.array_equal(got[guard:-guard], want)
    assert (got[:guard] == -1).all() and (got[-guard:] == -1).all()


def test_stream_probe_empty_is_a_no_op(device):
    e = torch.empty(0, dtype=torch.int32, device=device)
    probes.mhc_stream_probe(e, e, 5, 4)
    torch.cuda.synchronize()


@pytest.mark.parametrize("reads,writes", [(5, 4), (8, 0), (0, 8)])
@pytest.mark.parametrize("waves_per_block", [1, 4, 16])
@pytest.mark.parametrize("units", [1, 5, 300])
def test_clock_probe_moves_the_same_bytes_and_stamps_every_wave(device, reads, writes,
                                                                waves_per_block, units):
    say(f"clock probe {reads}:{writes} waves_per_block={waves_per_block} units={units}")
    rng = np.random.default_rng(reads * 100 + writes + units + 7 * waves_per_block)
    src_words = rng.integers(0, 2**32, size=units * reads * KiB // 4,
                             dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(src_words.view(np.int32)).to(device) if reads else None
    guard = 4096
    buf = torch.full((units * writes * KiB // 4 + 2 * guard,), -1, dtype=torch.int32,
                     device=device)
    dst = buf[guard:guard + units * writes * KiB // 4] if writes else None
    stamps = torch.full((4 * units + 64,), -1, dtype=torch.int64, device=device)
    probes.mhc_clock_probe(src, dst, reads, writes, waves_per_block, stamps)
    torch.cuda.synchronize()
    got = buf.cpu().numpy().view(np.uint32)
    if writes:
        want = (expected(src_words, reads, writes) if reads else
                np.repeat(np.arange(units, dtype=np.uint32), writes * KiB // 4))
        assert np.array_equal(got[guard:-guard], want)
    assert (got[:guard] == 0xFFFFFFFF).all() and (got[-guard:] == 0xFFFFFFFF).all()
    s = stamps.cpu().numpy()
    assert (s[4 * units:] == -1).all()
    s = s[:4 * units].reshape(units, 4)
    assert (s[:, 0] > 0).all()
    assert (s[:, 0] <= s[:, 1]).all() and (s[:, 1] <= s[:, 2]).all()
    assert ((s[:, 3] & 0xFFFFFFFF) < 16).all()
    # a wave's clock readings span at most a second
    assert ((s[:, 2] - s[:, 0]) < probes.mhc_probe_wall_clock_khz(device) * 1000).all()


def test_wall_clock_rate_is_known(device):
    assert probes.mhc_probe_wall_clock_khz(device) > 0

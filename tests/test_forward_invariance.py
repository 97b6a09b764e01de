"""forward_invariance: the forward's bytes never depend on the batch, the
partition or the launch shape.

The checks mirror the page "Add batch-invariant h_aggregate kernel" (RL-Kernel
pull request 366), section Correctness: 100 repeated calls are
byte-identical, and a full T=129 batch equals 129 one-token calls made with a
different launch shape. Added here: every launch-shape override, and canary
buffers showing each output element has exactly one writer and nothing
outside the output is written.
"""

from __future__ import annotations

import itertools

import numpy as np
import pytest
import torch

from conftest import assert_bytes_equal
from gpu_util import GUARD, SENTINELS, guarded_empty_bf16, guards_untouched, run_fwd, say
from hyper_connection_residual_mhc_amd import ops
from hyper_connection_residual_mhc_amd.workloads import bf16_tensor_to_bits, make_inputs, to_device
from oracle import h_aggregate as O

pytestmark = pytest.mark.gpu


def test_forward_100_repeats_byte_identical(device):
    say("forward 100 repeats T=129 H=4096")
    host = make_inputs(129, 4096, seed=0)
    d = to_device(host, device)
    outs = torch.empty((100, 129, 4096), dtype=torch.bfloat16, device=device)
    for k in range(100):
        ops.mhc_h_aggregate_fwd(d["residual"], d["pre"], outs[k])
    torch.cuda.synchronize()
    bits = outs.view(torch.int16)
    assert bool((bits == bits[0:1]).all())
    assert_bytes_equal(bf16_tensor_to_bits(outs[0]), O.h_aggregate_fwd(host["residual"], host["pre"]),
                       "forward T=129")


@pytest.mark.parametrize("T,H", [(129, 4096), (3, 1279)])
def test_forward_full_batch_equals_one_token_calls(device, T, H):
    """One call over T tokens (default launch: 64-thread blocks) vs T calls of
    one token each made with 1024-thread blocks, as in the page's check
    (different block size and partition), addressed by pointer offsets into
    the same buffers. The bytes must not change."""
    say(f"forward batch split T={T} H={H}")
    host = make_inputs(T, H, seed=1)
    d = to_device(host, device)
    full = torch.empty((T, H), dtype=torch.bfloat16, device=device)
    ops.mhc_h_aggregate_fwd(d["residual"], d["pre"], full)
    split = torch.empty((T, H), dtype=torch.bfloat16, device=device)
    for t in range(T):
        ops.mhc_h_aggregate_fwd(d["residual"][t:t + 1], d["pre"][t:t + 1], split[t:t + 1],
                                launch={"block_threads": 1024})
    torch.cuda.synchronize()
    plan_full, _ = ops.mhc_h_aggregate_plan_fwd(d["residual"], d["pre"], full, T, H)
    assert plan_full["block_threads"] != 1024
    assert_bytes_equal(bf16_tensor_to_bits(split), bf16_tensor_to_bits(full), "batch split")


def test_forward_uneven_batch_splits(device):
    """Splits of a 2048-token batch into 1, 7, 129 and the rest."""
    T, H = 2048, 7168
    say(f"forward uneven split T={T} H={H}")
    host = make_inputs(T, H, seed=2)
    d = to_device(host, device)
    full = torch.empty((T, H), dtype=torch.bfloat16, device=device)
    ops.mhc_h_aggregate_fwd(d["residual"], d["pre"], full)
    split = torch.empty_like(full)
    lo = 0
    for n in (1, 7, 129, T - 137):
        ops.mhc_h_aggregate_fwd(d["residual"][lo:lo + n], d["pre"][lo:lo + n], split[lo:lo + n])
        lo += n
    torch.cuda.synchronize()
    assert_bytes_equal(bf16_tensor_to_bits(split), bf16_tensor_to_bits(full), "uneven split")


@pytest.mark.parametrize("T,H", [(129, 4096), (7, 4104), (3, 1279)])
def test_forward_every_launch_shape_gives_the_same_bytes(device, T, H):
    host = make_inputs(T, H, seed=4)
    want = O.h_aggregate_fwd(host["residual"], host["pre"])
    widths = [v for v in (1, 2, 4, 8) if H % v == 0]
    for block, v, upt in itertools.product((64, 128, 192, 256, 512, 1024), widths, (1, 2, 4)):
        launch = {"block_threads": block, "vec_width": v, "units_per_thread": upt}
        say(f"forward launch {launch} T={T} H={H}")
        assert_bytes_equal(run_fwd(host, device, launch=launch), want, f"launch {launch}")


def test_forward_canaries_one_writer_and_no_stray_writes(device):
    """Outputs pre-filled with two different sentinel patterns come out with
    identical bytes (every element written), and the guard regions on both
    sides keep their sentinel (nothing written outside the output)."""
    T, H = 65, 1000
    host = make_inputs(T, H, seed=5)
    d = to_device(host, device)
    results = []
    for s in SENTINELS:
        for launch in (None, {"block_threads": 64, "vec_width": 2}, {"vec_width": 1}):
            say(f"forward canary sentinel=0x{s:x} launch={launch}")
            view, buf = guarded_empty_bf16((T, H), device, s)
            ops.mhc_h_aggregate_fwd(d["residual"], d["pre"], view, launch=launch)
            torch.cuda.synchronize()
            assert guards_untouched(buf, T * H, s)
            results.append(bf16_tensor_to_bits(view))
    for r in results[1:]:
        assert np.array_equal(r, results[0])
    assert_bytes_equal(results[0], O.h_aggregate_fwd(host["residual"], host["pre"]), "canary")
    assert GUARD > 0


def test_forward_concurrent_streams_same_bytes(device):
    """The same call on two streams at once (no shared state in the library)."""
    host = make_inputs(256, 4096, seed=6)
    d = to_device(host, device)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    o1 = torch.empty((256, 4096), dtype=torch.bfloat16, device=device)
    o2 = torch.empty_like(o1)
    torch.cuda.synchronize()
    say("forward two streams")
    for _ in range(10):
        ops.mhc_h_aggregate_fwd(d["residual"], d["pre"], o1, stream=s1)
        ops.mhc_h_aggregate_fwd(d["residual"], d["pre"], o2, stream=s2)
    torch.cuda.synchronize()
    assert_bytes_equal(bf16_tensor_to_bits(o1), bf16_tensor_to_bits(o2), "two streams")

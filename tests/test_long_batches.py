"""Batches longer than one dispatch can hold.

The forward's grid carries tokens in its y dimension (at most 65,535 per
dispatch), so a longer batch is split over several dispatches of whole
tokens; the results must not change, and a timed call's events must span
the first dispatch's start and the last one's end. The backward at the same
length runs as one dispatch per layout; it is checked the same way. The
oracle checks a sample of tokens (they are independent): both ends of the
batch, both sides of the dispatch boundary and 256 others."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from conftest import assert_bytes_equal
from gpu_util import HipEvents, say
from hyper_connection_residual_mhc_amd import ops
from hyper_connection_residual_mhc_amd.workloads import bf16_tensor_to_bits, make_inputs, to_device
from oracle import h_aggregate as O

pytestmark = pytest.mark.gpu

T_LONG = 70_001  # 65,535 + 4,466 tokens: two forward dispatches


def sample_tokens() -> np.ndarray:
    """Tokens to check against the oracle (tokens are independent): both ends
    of the batch, both sides of the dispatch boundary, and 256 others."""
    edges = np.concatenate([np.arange(0, 64), np.arange(65_535 - 64, 65_535 + 64),
                            np.arange(T_LONG - 64, T_LONG)])
    rest = np.random.default_rng(7).choice(T_LONG, 256, replace=False)
    return np.unique(np.concatenate([edges, rest]))


def subset(host: dict, toks: np.ndarray) -> dict:
    return {k: v[toks] for k, v in host.items()}


@pytest.mark.parametrize("H", [64, 136])
def test_forward_over_two_dispatches(device, H):
    say(f"long forward T={T_LONG} H={H}")
    host = make_inputs(T_LONG, H, seed=50 + H)
    d = to_device(host, device)
    plan, grid = ops.mhc_h_aggregate_plan_fwd(d["residual"], d["pre"], 1 << 40, T_LONG, H)
    assert grid == T_LONG * (-(-H // (plan["vec_width"] * plan["block_threads"])))
    out = torch.empty((T_LONG, H), dtype=torch.bfloat16, device=device)
    ev = HipEvents(2)
    try:
        ops.mhc_h_aggregate_fwd_timed(d["residual"], d["pre"], out, ev.h[0], ev.h[1])
        torch.cuda.synchronize()
        assert 0 < ev.elapsed_ms(0, 1) < 1000
    finally:
        ev.close()
    toks = sample_tokens()
    sub = subset(host, toks)
    assert_bytes_equal(bf16_tensor_to_bits(out)[toks], O.h_aggregate_fwd(sub["residual"], sub["pre"]),
                       f"forward T={T_LONG}")


@pytest.mark.parametrize("n", [2, 8])
def test_forward_n_over_two_dispatches(device, n):
    H = 64
    say(f"long forward n={n} T={T_LONG} H={H}")
    host = make_inputs(T_LONG, H, seed=60 + n, hc=n)
    d = to_device(host, device)
    out = torch.empty((T_LONG, H), dtype=torch.bfloat16, device=device)
    ops.mhc_h_aggregate_fwd_n(d["residual"], d["pre"], out)
    torch.cuda.synchronize()
    toks = sample_tokens()
    sub = subset(host, toks)
    assert_bytes_equal(bf16_tensor_to_bits(out)[toks],
                       O.h_aggregate_fwd_n(sub["residual"], sub["pre"]), f"forward n={n}")


@pytest.mark.parametrize("layout", [1, 2])
def test_backward_long_batch(device, layout):
    H = 64
    say(f"long backward T={T_LONG} H={H} layout={layout}")
    host = make_inputs(T_LONG, H, seed=70 + layout, grad=True)
    d = to_device(host, device)
    gr = torch.empty((T_LONG, 4, H), dtype=torch.bfloat16, device=device)
    gp = torch.empty((T_LONG, 4), dtype=torch.float32, device=device)
    ops.mhc_h_aggregate_bwd(d["residual"], d["pre"], d["grad_out"], gr, gp,
                            launch={"layout": layout})
    torch.cuda.synchronize()
    toks = sample_tokens()
    sub = subset(host, toks)
    want_gr, want_gp = O.h_aggregate_bwd(sub["residual"], sub["pre"], sub["grad_out"])
    assert_bytes_equal(bf16_tensor_to_bits(gr)[toks], want_gr, "grad_residual")
    assert_bytes_equal(gp.cpu().numpy()[toks], want_gp, "grad_pre")
    assert np.isfinite(gp.cpu().numpy()).all()

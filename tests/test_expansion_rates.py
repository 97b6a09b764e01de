"""Expansion rates 2 and 8 through mhc_h_aggregate_fwd_n / _bwd_n.

The page "Add batch-invariant h_aggregate kernel" (RL-Kernel pull request 366)
fixes 4 residual streams; the sibling mHC implementation of the second page
("perf: fuse mHC coefficient backward epilogue", Testing Done) covers HC in
{2, 4, 8}. Reading: the forward sums the n products as a balanced pairwise
tree ((0+1)+(2+3) at n = 4), the backward is per stream. The oracle is
oracle.h_aggregate_fwd_n / h_aggregate_bwd / h_aggregate_bwd_acc; tolerance
0 ulp.
"""

from __future__ import annotations

import itertools

import numpy as np
import pytest
import torch

from conftest import assert_bytes_equal
from gpu_util import say
from hyper_connection_residual_mhc_amd import ops
from hyper_connection_residual_mhc_amd.workloads import (bf16_tensor_to_bits, bits_to_bf16_tensor,
                                                         make_inputs, to_device)
from oracle import h_aggregate as O

pytestmark = pytest.mark.gpu


def fwd_n(host, dev, launch=None):
    d = to_device({"residual": host["residual"], "pre": host["pre"]}, dev)
    T, _, H = host["residual"].shape
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ops.mhc_h_aggregate_fwd_n(d["residual"], d["pre"], out, launch=launch)
    torch.cuda.synchronize()
    return bf16_tensor_to_bits(out)


def bwd_n(host, dev, old=None, launch=None):
    d = to_device(host, dev)
    T, n, H = host["residual"].shape
    if old is None:
        gr = torch.empty((T, n, H), dtype=torch.bfloat16, device=dev)
    else:
        gr = bits_to_bf16_tensor(old, dev).contiguous()
    gp = torch.empty((T, n), dtype=torch.float32, device=dev)
    ops.mhc_h_aggregate_bwd_n(d["residual"], d["pre"], d["grad_out"], gr, gp,
                              accumulate=old is not None, launch=launch)
    torch.cuda.synchronize()
    return bf16_tensor_to_bits(gr), gp.cpu().numpy()


SHAPES = [(1, 4096), (8, 7168), (129, 4096), (1024, 7168), (3, 1279), (6, 4100)]


@pytest.mark.parametrize("n", [2, 8])
@pytest.mark.parametrize("T,H", SHAPES)
def test_forward_n_bit_exact(device, n, T, H):
    say(f"forward n={n} T={T} H={H}")
    host = make_inputs(T, H, seed=T + H + n, hc=n, outliers=True)
    assert_bytes_equal(fwd_n(host, device), O.h_aggregate_fwd_n(host["residual"], host["pre"]),
                       f"forward n={n}")


@pytest.mark.parametrize("n", [2, 8])
@pytest.mark.parametrize("T,H", SHAPES)
def test_backward_n_bit_exact(device, n, T, H):
    say(f"backward n={n} T={T} H={H}")
    host = make_inputs(T, H, seed=T + H + 7 * n, hc=n, grad=True)
    gr, gp = bwd_n(host, device)
    want_gr, want_gp = O.h_aggregate_bwd(host["residual"], host["pre"], host["grad_out"])
    assert_bytes_equal(gr, want_gr, f"grad_residual n={n}")
    assert_bytes_equal(gp, want_gp, f"grad_pre n={n}")


@pytest.mark.parametrize("n", [2, 8])
@pytest.mark.parametrize("T", [300, 1031])
def test_backward_n_accumulate_bit_exact(device, n, T):
    H = 7168
    say(f"accumulate n={n}")
    host = make_inputs(T, H, seed=70 + n, hc=n, grad=True)
    old = make_inputs(T, H, seed=71 + n, hc=n)["residual"]
    gr, gp = bwd_n(host, device, old=old)
    want_gr, want_gp = O.h_aggregate_bwd_acc(host["residual"], host["pre"], host["grad_out"], old)
    assert_bytes_equal(gr, want_gr, f"accumulated n={n}")
    assert_bytes_equal(gp, want_gp, f"grad_pre n={n}")


def test_generic_entry_points_at_four_equal_the_page_ones(device):
    say("n=4 through the generic entry points")
    host = make_inputs(200, 7168, seed=80, grad=True)
    d = to_device(host, device)
    a = ops.h_aggregate(d["residual"], d["pre"])
    b = torch.empty_like(a)
    ops.mhc_h_aggregate_fwd_n(d["residual"], d["pre"], b)
    gr1, gp1 = ops.h_aggregate_backward(d["residual"], d["pre"], d["grad_out"])
    gr2, gp2 = torch.empty_like(gr1), torch.empty_like(gp1)
    ops.mhc_h_aggregate_bwd_n(d["residual"], d["pre"], d["grad_out"], gr2, gp2)
    torch.cuda.synchronize()
    assert_bytes_equal(bf16_tensor_to_bits(b), bf16_tensor_to_bits(a), "forward")
    assert_bytes_equal(bf16_tensor_to_bits(gr2), bf16_tensor_to_bits(gr1), "grad_residual")
    assert_bytes_equal(gp2.cpu().numpy(), gp1.cpu().numpy(), "grad_pre")


@pytest.mark.parametrize("n", [2, 8])
def test_n_every_launch_shape_same_bytes(device, n):
    T, H = 37, 4104
    host = make_inputs(T, H, seed=90 + n, hc=n, grad=True)
    want_out = O.h_aggregate_fwd_n(host["residual"], host["pre"])
    want_gr, want_gp = O.h_aggregate_bwd(host["residual"], host["pre"], host["grad_out"])
    for block, v in itertools.product((64, 256, 1024), (2, 4, 8)):
        for upt in (1, 2, 4):
            launch = {"block_threads": block, "vec_width": v, "units_per_thread": upt}
            try:
                ops.mhc_h_aggregate_plan_fwd_n(1 << 34, 1 << 35, 1 << 36, T, n, H, launch=launch)
            except Exception:
                continue   # beyond the register budget
            say(f"forward n={n} {launch}")
            assert_bytes_equal(fwd_n(host, device, launch), want_out, f"forward {launch}")
    for v, spb, tpb in itertools.product((2, 4, 8), (1, 2, 4), (1, 3)):
        if spb > n:
            continue
        launch = {"vec_width": v, "streams_per_block": spb, "tokens_per_block": tpb}
        say(f"backward n={n} {launch}")
        gr, gp = bwd_n(host, device, launch=launch)
        assert_bytes_equal(gr, want_gr, f"grad_residual {launch}")
        assert_bytes_equal(gp, want_gp, f"grad_pre {launch}")
    old = make_inputs(T, H, seed=99 + n, hc=n)["residual"]
    want_acc_gr, want_acc_gp = O.h_aggregate_bwd_acc(host["residual"], host["pre"],
                                                     host["grad_out"], old)
    for v, bt, prio in itertools.product((2, 4, 8), (64, 128, 256, 512), (1, 2)):
        if prio == 2 and v != 8:
            continue   # progress priority needs 16-byte accesses
        launch = {"layout": 2, "vec_width": v, "block_threads": bt, "wave_priority": prio}
        say(f"backward n={n} {launch}")
        gr, gp = bwd_n(host, device, launch=launch)
        assert_bytes_equal(gr, want_gr, f"grad_residual {launch}")
        assert_bytes_equal(gp, want_gp, f"grad_pre {launch}")
        gr, gp = bwd_n(host, device, old=old, launch=launch)
        assert_bytes_equal(gr, want_acc_gr, f"accumulated grad_residual {launch}")
        assert_bytes_equal(gp, want_acc_gp, f"accumulated grad_pre {launch}")


@pytest.mark.parametrize("n", [2, 8])
def test_n_batch_split(device, n):
    T, H = 160, 7168
    say(f"batch split n={n}")
    host = make_inputs(T, H, seed=95 + n, hc=n, grad=True)
    d = to_device(host, device)
    full = torch.empty((T, H), dtype=torch.bfloat16, device=device)
    ops.mhc_h_aggregate_fwd_n(d["residual"], d["pre"], full)
    split = torch.empty_like(full)
    gr = torch.empty((T, n, H), dtype=torch.bfloat16, device=device)
    gp = torch.empty((T, n), dtype=torch.float32, device=device)
    lo = 0
    for m in (1, 7, 129, 23):
        sl = slice(lo, lo + m)
        ops.mhc_h_aggregate_fwd_n(d["residual"][sl], d["pre"][sl], split[sl])
        ops.mhc_h_aggregate_bwd_n(d["residual"][sl], d["pre"][sl], d["grad_out"][sl], gr[sl], gp[sl])
        lo += m
    torch.cuda.synchronize()
    assert_bytes_equal(bf16_tensor_to_bits(split), bf16_tensor_to_bits(full), "forward split")
    want_gr, want_gp = O.h_aggregate_bwd(host["residual"], host["pre"], host["grad_out"])
    assert_bytes_equal(bf16_tensor_to_bits(gr), want_gr, "grad_residual split")
    assert_bytes_equal(gp.cpu().numpy(), want_gp, "grad_pre split")


@pytest.mark.parametrize("n", [2, 8])
def test_autograd_and_allocating_calls_at_n(device, n):
    """h_aggregate / h_aggregate_backward / HAggregate at expansion n: the
    same bytes as the oracle."""
    say(f"autograd n={n}")
    T, H = 16, 4096
    host = make_inputs(T, H, seed=40 + n, hc=n, grad=True)
    d = to_device(host, device)
    want_out = O.h_aggregate_fwd_n(host["residual"], host["pre"])
    want_gr, want_gp = O.h_aggregate_bwd(host["residual"], host["pre"], host["grad_out"])
    assert_bytes_equal(bf16_tensor_to_bits(ops.h_aggregate(d["residual"], d["pre"])), want_out,
                       f"h_aggregate n={n}")
    gr, gp = ops.h_aggregate_backward(d["residual"], d["pre"], d["grad_out"])
    torch.cuda.synchronize()
    assert_bytes_equal(bf16_tensor_to_bits(gr), want_gr, f"h_aggregate_backward n={n} grad_residual")
    assert_bytes_equal(gp.cpu().numpy(), want_gp, f"h_aggregate_backward n={n} grad_pre")
    res = d["residual"].clone().requires_grad_(True)
    pre = d["pre"].clone().requires_grad_(True)
    out = ops.h_aggregate_autograd(res, pre)
    out.backward(d["grad_out"])
    torch.cuda.synchronize()
    assert_bytes_equal(bf16_tensor_to_bits(out), want_out, f"autograd n={n} out")
    assert_bytes_equal(bf16_tensor_to_bits(res.grad), want_gr, f"autograd n={n} grad_residual")
    assert_bytes_equal(pre.grad.cpu().numpy(), want_gp, f"autograd n={n} grad_pre")

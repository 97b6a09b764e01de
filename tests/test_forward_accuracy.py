"""forward_accuracy: the gfx950 forward against the CPU oracle, bit for bit.

Operation: page "Add batch-invariant h_aggregate kernel" (RL-Kernel pull
request 366), Summary (formula, shapes) and Batch invariance (fp32
round-to-nearest mul/add, fixed tree, one bf16 rounding). Tolerance: 0 ulp
(every output byte equal). Workloads: the shapes of the page's Correctness
and Performance sections, with the seeded synthetic inputs of
hyper_connection_residual_mhc_amd.workloads.
"""

from __future__ import annotations

import json
from pathlib import Path

import numpy as np
import pytest
import torch

from conftest import assert_bytes_equal
from gpu_util import offset_copy_bf16, run_fwd, say
from hyper_connection_residual_mhc_amd import ops
from hyper_connection_residual_mhc_amd.workloads import (bf16_tensor_to_bits, make_inputs,
                                                         to_device)
from oracle import h_aggregate as O

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,H", [(8, 4096),                                    # small case
                                 (1, 4096), (8, 4096), (128, 4096),            # latency sweep
                                 (1, 7168), (8, 7168), (128, 7168),
                                 (129, 4096), (3, 1279)])                      # invariance shapes
def test_forward_bit_exact_page_shapes(device, T, H):
    say(f"forward parity T={T} H={H}")
    host = make_inputs(T, H, seed=0)
    assert_bytes_equal(run_fwd(host, device), O.h_aggregate_fwd(host["residual"], host["pre"]),
                       f"forward T={T} H={H}")


@pytest.mark.parametrize("H", [1, 2, 3, 4, 5, 7, 8, 9, 12, 63, 64, 65, 100, 1276, 1278, 1279,
                               4104, 7169, 8200])
def test_forward_bit_exact_ragged_hidden_sizes(device, H):
    """Every vector width (H % 8, 4, 2 and odd) and ragged block tails."""
    say(f"forward ragged H={H}")
    host = make_inputs(5, H, seed=H)
    assert_bytes_equal(run_fwd(host, device), O.h_aggregate_fwd(host["residual"], host["pre"]),
                       f"forward H={H}")


def test_forward_bit_exact_bandwidth_shape_with_outliers(device):
    """T=1024, H=7168 with 1% x64 outliers: every element, plus the fp64 gate."""
    say("forward parity T=1024 H=7168 outliers")
    host = make_inputs(1024, 7168, seed=0, outliers=True)
    got = run_fwd(host, device)
    assert_bytes_equal(got, O.h_aggregate_fwd(host["residual"], host["pre"]), "forward T=1024")
    exact, mag = O.h_aggregate_fwd_exact(host["residual"], host["pre"])
    c = O.classify_fwd(got, exact, mag)
    assert c["fail"] == 0, c


def test_forward_large_batch_every_token(device):
    """T=8192, H=7168 (the largest bandwidth shape, with 1% x64 outliers),
    run in one call; every token compared with the oracle byte for byte,
    1024 tokens at a time (the oracle is per token), and every output within
    the fp64 gate."""
    T, H = 8192, 7168
    say(f"forward parity T={T} H={H} every token")
    host = make_inputs(T, H, seed=0, outliers=True)
    got = run_fwd(host, device)
    for lo in range(0, T, 1024):
        r, p = host["residual"][lo:lo + 1024], host["pre"][lo:lo + 1024]
        assert_bytes_equal(got[lo:lo + 1024], O.h_aggregate_fwd(r, p),
                           f"forward T={T} tokens {lo}..{lo + 1023}")
        exact, mag = O.h_aggregate_fwd_exact(r, p)
        assert O.classify_fwd(got[lo:lo + 1024], exact, mag)["fail"] == 0


def test_forward_golden_vectors_on_device(device):
    """The hand-derived cases (denormal kept, signed zeros, overflow, no FMA,
    the tree discriminator) through the kernel, 8 copies wide so that the
    16-byte vector path handles them too."""
    doc = json.loads((Path(__file__).parent / "golden" / "forward_hand_vectors.json").read_text())
    for case in doc["cases"]:
        say(f"forward golden {case['name']}")
        pre = np.array([int(p, 16) for p in case["pre_bits"]], np.uint32).view(np.float32)
        res = np.array([int(r, 16) for r in case["residual_bits"]], np.uint16)
        for H in (1, 8):
            host = {"residual": np.repeat(res[None, :, None], H, axis=2).copy(),
                    "pre": pre.reshape(1, 4).copy()}
            got = run_fwd(host, device)
            assert (got == int(case["out_bits"], 16)).all(), (case["name"], H, got)


def test_forward_special_values(device):
    """Subnormal-range products, huge values that overflow, zeros of both
    signs, infinities: bit-exact against the oracle for finite inputs, NaN
    where the oracle gives NaN."""
    rng = np.random.default_rng(21)
    T, H = 16, 1024
    mags = np.exp2(rng.integers(-140, 128, (T, 4, H))).astype(np.float64)
    vals = (rng.standard_normal((T, 4, H)) * mags)
    with np.errstate(over="ignore"):
        f = vals.astype(np.float32)
    f[0, :, :8] = 0.0
    f[1, :, :8] = -0.0
    f[2, 0, :4] = np.inf
    f[2, 1, 4:8] = -np.inf
    from hyper_connection_residual_mhc_amd.workloads import to_bf16_bits
    host = {"residual": to_bf16_bits(f),
            "pre": np.exp2(rng.integers(-30, 30, (T, 4))).astype(np.float32)}
    host["pre"][3] = [2.0 ** -126, 2.0 ** -149, 1e-40, 3e38]
    got = run_fwd(host, device)
    want = O.h_aggregate_fwd(host["residual"], host["pre"])
    nan_w = np.isnan(O.widen_bf16(want))
    assert np.array_equal(np.isnan(O.widen_bf16(got)), nan_w)
    assert_bytes_equal(got[~nan_w], want[~nan_w], "forward special values")


def test_forward_misaligned_buffers_narrow_the_vector_only(device):
    """Offsetting residual or out by 1, 2 or 3 elements forces the 8/4/2-byte
    or scalar paths; the bytes are the same as the aligned call's."""
    T, H = 17, 4096
    host = make_inputs(T, H, seed=3)
    want = O.h_aggregate_fwd(host["residual"], host["pre"])
    pre = torch.from_numpy(host["pre"]).to(device)
    for off_r, off_o in ((1, 0), (2, 0), (4, 0), (0, 1), (0, 2), (3, 5)):
        say(f"forward misaligned residual+{off_r} out+{off_o}")
        res = offset_copy_bf16(host["residual"], device, off_r)
        obuf = torch.empty(T * H + off_o, dtype=torch.bfloat16, device=device)
        out = obuf[off_o:].view(T, H)
        ops.mhc_h_aggregate_fwd(res, pre, out)
        torch.cuda.synchronize()
        assert_bytes_equal(bf16_tensor_to_bits(out), want, f"misaligned {off_r},{off_o}")


def test_forward_empty_batch_is_a_no_op(device):
    say("forward T=0")
    res = torch.empty((0, 4, 4096), dtype=torch.bfloat16, device=device)
    pre = torch.empty((0, 4), dtype=torch.float32, device=device)
    out = torch.empty((0, 4096), dtype=torch.bfloat16, device=device)
    ops.mhc_h_aggregate_fwd(res, pre, out)
    torch.cuda.synchronize()


def test_forward_matches_torch_reference_within_page_tolerance(device):
    """The page's own check: a PyTorch reference at atol 5e-2, rtol 1e-2
    (computed in fp32 on the GPU, then bf16)."""
    say("forward vs torch reference")
    host = make_inputs(128, 7168, seed=1)
    d = to_device(host, device)
    out = ops.h_aggregate(d["residual"], d["pre"]).float()
    ref = (d["pre"][:, :, None] * d["residual"].float()).sum(dim=1).to(torch.bfloat16).float()
    torch.testing.assert_close(out, ref, atol=5e-2, rtol=1e-2)


def test_page_entry_point_name_runs_the_kernel(device):
    """mhc_pre_h_aggregate (the name the page's tests call) gives the
    oracle's bytes, at the page's correctness shape T=129, H=4096."""
    say("mhc_pre_h_aggregate")
    host = make_inputs(129, 4096, seed=3)
    d = to_device(host, device)
    got = bf16_tensor_to_bits(ops.mhc_pre_h_aggregate(d["residual"], d["pre"]))
    assert_bytes_equal(got, O.h_aggregate_fwd(host["residual"], host["pre"]), "entry point")

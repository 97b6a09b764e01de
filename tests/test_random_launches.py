"""Seeded random cases on the GPU: shape (T, H), expansion rate n, and a
launch override drawn among the fields the plan accepts for it (layout,
vector width, ring or units, block size, tokens and streams per block, issue
priority). Forward, written backward and accumulating backward, each byte
for byte against the oracle. Complements the grid sweeps of the invariance
tests with combinations they do not enumerate."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from conftest import assert_bytes_equal
from gpu_util import say
from hyper_connection_residual_mhc_amd import ops
from hyper_connection_residual_mhc_amd._lib import MhcError
from hyper_connection_residual_mhc_amd.workloads import (bf16_tensor_to_bits, bits_to_bf16_tensor,
                                                         make_inputs, to_device)
from oracle import h_aggregate as O

pytestmark = pytest.mark.gpu

CASES = 48
FAKE = (1 << 34, 1 << 35, 1 << 36, 1 << 37, 1 << 38)   # plan queries only read addresses


def draw_case(rng: np.random.Generator) -> dict:
    n = int(rng.choice([2, 4, 8]))
    T = int(rng.integers(1, 97))
    if rng.random() < 0.5:
        H = int(rng.integers(1, 64)) * 8 * int(rng.choice([1, 16]))     # multiples of 8
    else:
        H = int(rng.integers(1, 9000))                                 # any width
    H = max(1, min(H, 9000))
    bwd = {}
    if rng.random() < 0.5:
        bwd["layout"] = 2
        bwd["units_per_thread"] = int(rng.choice([4, 8, 12]))
        bwd["block_threads"] = int(rng.choice([64, 128, 256, 512]))
        bwd["wave_priority"] = int(rng.choice([1, 2]))
    else:
        bwd["layout"] = 1
        bwd["units_per_thread"] = int(rng.choice([1, 2, 4]))
        bwd["tokens_per_block"] = int(rng.choice([1, 2, 3, 5]))
        bwd["streams_per_block"] = int(rng.choice([s for s in (1, 2, 4) if s <= n]))
    if rng.random() < 0.5:
        bwd["vec_width"] = int(rng.choice([v for v in (1, 2, 4, 8) if H % v == 0]))
    fwd = {"block_threads": int(rng.choice([64, 128, 256, 1024])),
           "units_per_thread": int(rng.choice([1, 2, 4]))}
    return {"T": T, "H": H, "n": n, "bwd": bwd, "fwd": fwd, "seed": int(rng.integers(1 << 30))}


def accepted(plan_fn, *args, **kwargs) -> bool:
    """Whether the plan accepts the call (host-only query)."""
    try:
        plan_fn(*args, **kwargs)
        return True
    except MhcError:
        return False


@pytest.mark.parametrize("k", range(CASES))
def test_random_case_matches_the_oracle(device, k):
    rng = np.random.default_rng(1000 + k)
    c = draw_case(rng)
    T, H, n = c["T"], c["H"], c["n"]
    host = make_inputs(T, H, seed=c["seed"], hc=n, grad=True, outliers=True)
    d = to_device(host, device)
    fwd = c["fwd"] if accepted(ops.mhc_h_aggregate_plan_fwd_n, *FAKE[:3], T, n, H,
                               launch=c["fwd"]) else None
    bwd = c["bwd"] if accepted(ops.mhc_h_aggregate_plan_bwd_n, *FAKE, T, n, H,
                               launch=c["bwd"]) else None
    say(f"random case {k}: T={T} H={H} n={n} fwd={fwd} bwd={bwd}")

    out = torch.empty((T, H), dtype=torch.bfloat16, device=device)
    ops.mhc_h_aggregate_fwd_n(d["residual"], d["pre"], out, launch=fwd)
    gr = torch.empty((T, n, H), dtype=torch.bfloat16, device=device)
    gp = torch.empty((T, n), dtype=torch.float32, device=device)
    ops.mhc_h_aggregate_bwd_n(d["residual"], d["pre"], d["grad_out"], gr, gp, launch=bwd)
    old = make_inputs(T, H, seed=c["seed"] + 1, hc=n)["residual"]
    gra = bits_to_bf16_tensor(old, device).contiguous()
    gpa = torch.empty((T, n), dtype=torch.float32, device=device)
    acc_launch = bwd if bwd is not None and accepted(
        ops.mhc_h_aggregate_plan_bwd_n, *FAKE, T, n, H, launch=bwd, accumulate=True) else None
    ops.mhc_h_aggregate_bwd_n(d["residual"], d["pre"], d["grad_out"], gra, gpa, accumulate=True,
                              launch=acc_launch)
    torch.cuda.synchronize()

    assert_bytes_equal(bf16_tensor_to_bits(out), O.h_aggregate_fwd_n(host["residual"], host["pre"]),
                       f"case {k} forward")
    want_gr, want_gp = O.h_aggregate_bwd(host["residual"], host["pre"], host["grad_out"])
    assert_bytes_equal(bf16_tensor_to_bits(gr), want_gr, f"case {k} grad_residual")
    assert_bytes_equal(gp.cpu().numpy(), want_gp, f"case {k} grad_pre")
    want_gra, want_gpa = O.h_aggregate_bwd_acc(host["residual"], host["pre"], host["grad_out"], old)
    assert_bytes_equal(bf16_tensor_to_bits(gra), want_gra, f"case {k} accumulated grad_residual")
    assert_bytes_equal(gpa.cpu().numpy(), want_gpa, f"case {k} accumulated grad_pre")

"""The entry points inside a captured HIP graph.

The library only validates on the host and enqueues kernels (no allocation,
no memset, no synchronisation), so a stream capture of a forward and a
backward replays them as graph nodes. Each replay is checked against the
eager result, with other eager work and synchronisations between replays,
and the inputs are changed between replays to show the graph reads them
afresh.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from conftest import assert_bytes_equal
from gpu_util import say
from hyper_connection_residual_mhc_amd import ops
from hyper_connection_residual_mhc_amd.workloads import (bf16_tensor_to_bits, make_inputs,
                                                         to_device)
from oracle import h_aggregate as O

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,H", [(8, 4096), (1024, 7168)])
def test_forward_and_backward_replay_from_a_graph(device, T, H):
    say(f"graph capture T={T} H={H}")
    d = to_device(make_inputs(T, H, seed=40, grad=True), device)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=device)
    gr = torch.empty((T, 4, H), dtype=torch.bfloat16, device=device)
    gp = torch.empty((T, 4), dtype=torch.float32, device=device)
    acc = torch.zeros_like(gr)

    def step():
        ops.mhc_h_aggregate_fwd(d["residual"], d["pre"], out)
        ops.mhc_h_aggregate_bwd(d["residual"], d["pre"], d["grad_out"], gr, gp)
        ops.mhc_h_aggregate_bwd_acc(d["residual"], d["pre"], d["grad_out"], acc, gp)

    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for replay in range(4):
        say(f"graph replay {replay}")
        host = make_inputs(T, H, seed=41 + replay, grad=True)
        for k in ("residual", "pre", "grad_out"):
            d[k].copy_(to_device({k: host[k]}, device)[k])
        acc.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want_out = O.h_aggregate_fwd(host["residual"], host["pre"])
        want_gr, want_gp = O.h_aggregate_bwd(host["residual"], host["pre"], host["grad_out"])
        assert_bytes_equal(bf16_tensor_to_bits(out), want_out, f"replay {replay} forward")
        assert_bytes_equal(bf16_tensor_to_bits(gr), want_gr, f"replay {replay} grad_residual")
        assert_bytes_equal(gp.cpu().numpy(), want_gp, f"replay {replay} grad_pre")
        # the accumulating form onto +0 (the oracle applies the same reading)
        assert np.array_equal(bf16_tensor_to_bits(acc),
                              O.grad_residual_acc_ref(host["pre"], host["grad_out"],
                                                      np.zeros((T, 4, H), np.uint16)))
        # eager work between replays
        eager = ops.h_aggregate(d["residual"], d["pre"])
        torch.cuda.synchronize()
        assert torch.equal(eager.view(torch.int16), out.view(torch.int16))


@pytest.mark.parametrize("launches", [1, 2])
def test_coefficient_backward_replays_from_a_graph(device, launches):
    """The coefficient epilogue in a captured graph: its arrival counter is
    left at zero by every replay, so replays keep giving the oracle's bits."""
    from hyper_connection_residual_mhc_amd import coeff
    from hyper_connection_residual_mhc_amd.workloads import make_coeff_inputs
    from oracle import coeff_bwd as CB
    say(f"graph capture coefficient backward launches={launches}")
    keys = ("mix", "pre", "post", "grad_pre", "grad_post", "grad_res", "alpha")
    R, n = 2048, 4
    d = {k: torch.from_numpy(v).to(device) for k, v in make_coeff_inputs(R, n, seed=50).items()}
    gm = torch.empty((R, 24), dtype=torch.float32, device=device)
    gb = torch.empty((24,), dtype=torch.float32, device=device)
    ga = torch.empty((3,), dtype=torch.float32, device=device)
    ws = torch.zeros(coeff.mhc_coeff_bwd_workspace_bytes(R, n), dtype=torch.uint8, device=device)

    def step():
        coeff.mhc_coeff_bwd(*(d[k] for k in keys), 2.0, grad_mix=gm, grad_b=gb, grad_alpha=ga,
                            workspace=ws, launches=launches)

    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for replay in range(4):
        host = make_coeff_inputs(R, n, seed=51 + replay)
        for k in keys:
            d[k].copy_(torch.from_numpy(host[k]).to(device))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = CB.coeff_bwd(*(host[k] for k in keys), 2.0, n)
        for name, got, w in zip(("grad_mix", "grad_b", "grad_alpha"), (gm, gb, ga), want):
            assert_bytes_equal(got.cpu().numpy(), w, f"replay {replay} {name}")
        assert int(ws[:4].view(torch.int32).item()) == 0
        step()                                  # eager work between replays
        torch.cuda.synchronize()
        assert_bytes_equal(gb.cpu().numpy(), want[1], f"eager after replay {replay}")

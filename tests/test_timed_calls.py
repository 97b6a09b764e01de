"""The *_timed entry points: same bytes as the plain calls, and the events
they attach to the kernel dispatches bracket the kernels' execution."""

from __future__ import annotations

import pytest
import torch

from conftest import assert_bytes_equal
from gpu_util import HipEvents, run_bwd, run_fwd, say
from hyper_connection_residual_mhc_amd import ops
from hyper_connection_residual_mhc_amd.workloads import bf16_tensor_to_bits, make_inputs, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,H", [(1024, 7168), (3, 1279), (0, 64)])
def test_timed_calls_same_bytes_and_positive_times(device, T, H):
    say(f"timed calls T={T} H={H}")
    host = make_inputs(T, H, seed=1, grad=True)
    d = to_device(host, device)
    ev = HipEvents(4)
    try:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=device)
        ops.mhc_h_aggregate_fwd_timed(d["residual"], d["pre"], out, ev.h[0], ev.h[1])
        gr = torch.empty((T, 4, H), dtype=torch.bfloat16, device=device)
        gp = torch.empty((T, 4), dtype=torch.float32, device=device)
        ops.mhc_h_aggregate_bwd_timed(d["residual"], d["pre"], d["grad_out"], gr, gp,
                                      ev.h[2], ev.h[3])
        torch.cuda.synchronize()
        tf, tb = ev.elapsed_ms(0, 1), ev.elapsed_ms(2, 3)
        if T == 0:
            assert tf >= 0 and tb >= 0
            return
        assert 0 < tf < 100 and 0 < tb < 100, (tf, tb)
        assert_bytes_equal(bf16_tensor_to_bits(out), run_fwd(host, device), "timed forward")
        want_gr, want_gp = run_bwd(host, device)
        assert_bytes_equal(bf16_tensor_to_bits(gr), want_gr, "timed grad_residual")
        assert_bytes_equal(gp.cpu().numpy(), want_gp, "timed grad_pre")
    finally:
        ev.close()


def test_timed_call_with_only_one_event(device):
    say("timed call with one event")
    host = make_inputs(8, 4096, seed=2)
    d = to_device(host, device)
    ev = HipEvents(2)
    try:
        out = torch.empty((8, 4096), dtype=torch.bfloat16, device=device)
        ops.mhc_h_aggregate_fwd_timed(d["residual"], d["pre"], out, ev.h[0], None)
        ops.mhc_h_aggregate_fwd_timed(d["residual"], d["pre"], out, None, ev.h[1])
        torch.cuda.synchronize()
        assert ev.elapsed_ms(0, 1) > 0
    finally:
        ev.close()

"""The no-allocation entry point of the coefficient epilogue
(mhc_coeff_bwd_noalloc, include/mhc_coeff_bwd.h) against the workspace entry
point (mhc_coeff_bwd) and the oracle, bit for bit, through the C ABI.

Calls come in pairs, one after another on one stream with the second input
smaller than the first, so that the second call meets the scratch array as
the first left it (chunk sums of a longer batch, the arrival counter reset).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from conftest import assert_bytes_equal
from gpu_util import say
from hyper_connection_residual_mhc_amd import _lib
from hyper_connection_residual_mhc_amd.workloads import make_coeff_inputs
from oracle import coeff_bwd as cb

pytestmark = pytest.mark.gpu

KEYS = ("mix", "pre", "post", "grad_pre", "grad_post", "grad_res", "alpha")


def _device(host, dev):
    return {k: torch.from_numpy(np.ascontiguousarray(host[k])).to(dev) for k in KEYS}


def _outputs(R, n, dev):
    m = 2 * n + n * n
    return (torch.full((R, m), float("nan"), device=dev), torch.full((m,), float("nan"), device=dev),
            torch.full((3,), float("nan"), device=dev))


def _noalloc(d, outs, c, R, n, launches, sh):
    lib = _lib.coeff_lib()
    return lib.mhc_coeff_bwd_noalloc(*(d[k].data_ptr() for k in KEYS), c,
                                     *(o.data_ptr() for o in outs), R, n, launches, sh, None, None)


def _with_workspace(d, outs, c, R, n, launches, sh, dev):
    lib = _lib.coeff_lib()
    need = lib.mhc_coeff_bwd_workspace_bytes(R, n)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib.mhc_coeff_bwd(*(d[k].data_ptr() for k in KEYS), c, *(o.data_ptr() for o in outs),
                           ws.data_ptr(), need, R, n, launches, sh, None, None)
    return st, ws


@pytest.mark.parametrize("n,sizes", [(4, (8192, 1000)), (2, (20000, 65)), (8, (6000, 300)),
                                     (4, (1242560, 4097))])
@pytest.mark.parametrize("launches", [0, 1, 2])
def test_noalloc_matches_the_workspace_entry_point(device, n, sizes, launches):
    sh = int(torch.cuda.current_stream(device).cuda_stream)
    c = 2.0 if n != 2 else 3.0
    for R in sizes:                 # the second call is the smaller one
        say(f"coeff noalloc n={n} R={R} launches={launches}")
        host = make_coeff_inputs(R, n, seed=R + n, post_scale=c)
        d = _device(host, device)
        got, want = _outputs(R, n, device), _outputs(R, n, device)
        _lib.check_coeff(_noalloc(d, got, c, R, n, launches, sh))
        st, ws = _with_workspace(d, want, c, R, n, launches, sh, device)
        _lib.check_coeff(st)
        torch.cuda.synchronize()
        oracle = cb.coeff_bwd(*(host[k] for k in KEYS), c, n) if R <= 20000 else None
        for i, name in enumerate(("grad_mix", "grad_b", "grad_alpha")):
            g = got[i].cpu().numpy()
            assert_bytes_equal(g, want[i].cpu().numpy(), f"noalloc vs workspace {name} R={R}")
            if oracle is not None:
                assert_bytes_equal(g, oracle[i], f"noalloc vs oracle {name} R={R}")
        del ws


def test_noalloc_empty_batch_and_refusal(device):
    """R = 0 writes the +0.0 sums; a call past the scratch capacity is
    refused and leaves its outputs untouched."""
    sh = int(torch.cuda.current_stream(device).cuda_stream)
    say("coeff noalloc R=0 and too large")
    host = make_coeff_inputs(0, 4, seed=1)
    d = _device(host, device)
    outs = _outputs(0, 4, device)
    _lib.check_coeff(_noalloc(d, outs, 2.0, 0, 4, 0, sh))
    torch.cuda.synchronize()
    assert outs[1].cpu().tolist() == [0.0] * 24 and outs[2].cpu().tolist() == [0.0] * 3
    R = 1242560 + 1
    p = torch.empty(1, device=device)
    big = _outputs(1, 4, device)
    st = _lib.coeff_lib().mhc_coeff_bwd_noalloc(*([p.data_ptr()] * 7), 2.0,
                                                *(o.data_ptr() for o in big), R, 4, 0, sh,
                                                None, None)
    assert st == _lib.MHC_ERROR_INVALID_VALUE
    torch.cuda.synchronize()
    assert torch.isnan(big[0]).all() and torch.isnan(big[1]).all()

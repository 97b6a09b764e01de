"""The coefficient epilogue at the most rows it accepts (MHC_COEFF_MAX_ROWS
= 2^28) at n = 2: about 28 GiB on the device, 2^22 chunks, every workspace
offset at its largest.

grad_mix rows depend only on their own row, so sampled rows (both ends and
4,096 others) are checked against the oracle. The sums are made exact in any
order: grad_pre = grad_post = 0, mix = +-1 and grad_res = +-1 on 1/128 of its
entries (0 elsewhere), so every derivative, product and partial sum is an
integer whose magnitude is bounded by the number of non-zero terms (about
2^23, checked to be at most 2^24), and fp32 holds them exactly. grad_b and
grad_alpha must then equal integer sums formed on the host from the inputs'
codes. Both launch forms run."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from conftest import assert_bytes_equal
from gpu_util import say
from hyper_connection_residual_mhc_amd import _lib, coeff
from hyper_connection_residual_mhc_amd.workloads import make_coeff_unit_inputs_device
from oracle import coeff_bwd as cb

pytestmark = pytest.mark.gpu

R_MAX = _lib.MHC_COEFF_MAX_ROWS
N = 2
M = 2 * N + N * N
KEYS = ("mix", "pre", "post", "grad_pre", "grad_post", "grad_res", "alpha")


@pytest.fixture(scope="module")
def case(device):
    say(f"coeff max rows: building inputs R={R_MAX} n={N}")
    d = make_coeff_unit_inputs_device(R_MAX, N, 28, device)
    rows = np.unique(np.concatenate([np.arange(0, 64), np.arange(R_MAX - 64, R_MAX),
                                     np.random.default_rng(9).choice(R_MAX, 4096, replace=False)]))
    idx = torch.from_numpy(rows).to(device)
    sub = {k: d[k][idx].cpu().numpy() if k != "alpha" else d[k].cpu().numpy() for k in KEYS}
    # exact sums from the codes: d = grad_res on the residual columns, 0 elsewhere
    rc = d["grad_res_code"].cpu().numpy()
    dres = (rc == 1).astype(np.int8) - (rc == 0).astype(np.int8)      # [R, n*n]
    del rc
    assert np.count_nonzero(dres) <= 2 ** 24
    mc = d["mix_code"][:, 2 * N:].cpu().numpy()
    sgn = mc.astype(np.int8) * 2 - 1
    del mc
    grad_b = np.zeros(M, dtype=np.int64)
    grad_b[2 * N:] = dres.sum(axis=0, dtype=np.int64)
    alpha2 = int(np.sum(dres * sgn, dtype=np.int64))
    del dres, sgn
    del d["mix_code"], d["grad_res_code"]
    return d, sub, grad_b, alpha2


@pytest.mark.parametrize("launches", [2, 1])
def test_coefficient_backward_at_the_most_rows(case, device, launches):
    d, sub, grad_b, alpha2 = case
    say(f"coeff max rows: launches={launches}")
    gm, gb, ga = coeff.mhc_coeff_bwd(*(d[k] for k in KEYS), 2.0, launches=launches)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 64), np.arange(R_MAX - 64, R_MAX),
                                     np.random.default_rng(9).choice(R_MAX, 4096, replace=False)]))
    got_rows = gm[torch.from_numpy(rows).to(device)].cpu().numpy()
    want_rows = cb.coeff_bwd(*(sub[k] for k in KEYS), 2.0, N)[0]
    assert_bytes_equal(got_rows, want_rows, f"grad_mix sampled rows launches={launches}")
    assert np.array_equal(gb.cpu().numpy(), grad_b.astype(np.float32)), (gb.cpu(), grad_b)
    want_a = np.array([0.0, 0.0, float(alpha2)], dtype=np.float32)
    assert np.array_equal(ga.cpu().numpy(), want_a), (ga.cpu(), want_a)
    assert not torch.signbit(gb[:2 * N]).any() and not torch.signbit(ga[:2]).any()

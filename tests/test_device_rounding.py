"""The device's bf16 rounding against the oracle over all 2^32 fp32 patterns.

Every bf16 result of the kernels goes through one device routine (exposed as
mhc_bf16_rne_probe). Round to nearest even on a pattern (hi, lo) - hi the
top 16 bits, lo the bottom 16 - gives the same answer for every lo in
[0, 0x7FFF] and for every lo in [0x8001, 0xFFFF] (for finite hi). So the
device output over all 2^32 patterns equals the oracle's exactly when
(a) on the device, each hi row is constant on those two lo ranges, and
(b) at lo in {0, 0x7FFF, 0x8000, 0x8001, 0xFFFF} the device equals the oracle.
(a) is checked on the GPU for every row, (b) on the host for every row.
NaN inputs only need to give NaN (the page does not fix a NaN payload).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_util import say
from hyper_connection_residual_mhc_amd import probes
from oracle import h_aggregate as O

pytestmark = pytest.mark.gpu

ROWS_PER_CHUNK = 1 << 12            # 4096 hi values x 65536 lo = 2^28 patterns
REPS = np.array([0x0000, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)


def test_device_bf16_rounding_all_patterns(device):
    out = torch.empty(ROWS_PER_CHUNK << 16, dtype=torch.int16, device=device)
    for c in range((1 << 16) // ROWS_PER_CHUNK):
        hi0 = c * ROWS_PER_CHUNK
        say(f"rounding probe rows {hi0:#06x}..{hi0 + ROWS_PER_CHUNK - 1:#06x}")
        probes.mhc_bf16_rne_probe(hi0 << 16, out)
        rows = out.view(ROWS_PER_CHUNK, 1 << 16)
        hi = np.arange(hi0, hi0 + ROWS_PER_CHUNK, dtype=np.uint32)
        exp_all_ones = (hi & 0x7F80) == 0x7F80          # Inf / NaN rows
        low = rows[:, :0x8000]
        high = rows[:, 0x8001:]
        const_low = (low == low[:, :1]).all(dim=1).cpu().numpy()
        const_high = (high == high[:, :1]).all(dim=1).cpu().numpy()
        finite = ~exp_all_ones
        assert const_low[finite].all() and const_high[finite].all(), hex(hi0)
        reps = rows[:, torch.from_numpy(REPS.astype(np.int64)).to(device)].cpu().numpy().view(np.uint16)
        pats = (hi[:, None] << np.uint32(16)) | REPS[None, :]
        want = O.bf16_rne(pats.view(np.float32))
        fin = finite[:, None].repeat(len(REPS), 1)
        assert np.array_equal(reps[fin], want[fin]), hex(hi0)
        # Inf / NaN rows: lo == 0 is +-Inf exactly, every other lo is NaN.
        if exp_all_ones.any():
            sub = rows[torch.from_numpy(np.flatnonzero(exp_all_ones)).to(device)]
            wid = (sub.to(torch.int32) << 16).view(torch.float32)
            assert bool(torch.isnan(wid[:, 1:]).all())
            inf_rows = hi[exp_all_ones]
            inf_bits = sub[:, 0].cpu().numpy().view(np.uint16)
            assert np.array_equal(inf_bits[(inf_rows & 0x7F) == 0], (inf_rows[(inf_rows & 0x7F) == 0]).astype(np.uint16))
    torch.cuda.synchronize()

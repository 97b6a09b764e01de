"""The coefficient backward epilogue on the GPU against the oracle
(oracle/coeff_bwd.py), bit for bit, through the C ABI.

Shapes: the page "perf: fuse mHC coefficient backward epilogue" (Performance
Method) measures B = 4 sequences of T in {128, 512, 2048} tokens, i.e.
R = 512, 2048 and 8192 rows, at HC = 4 with HC = 2 and 8 as controls. The
other row counts span one chunk, a ragged chunk, several chunks and more
than 64 chunks (the second stage's strided walk).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from conftest import assert_bytes_equal
from gpu_util import HipEvents, say
from hyper_connection_residual_mhc_amd import coeff
from hyper_connection_residual_mhc_amd.workloads import make_coeff_inputs
from oracle import coeff_bwd as cb

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
KEYS = ("mix", "pre", "post", "grad_pre", "grad_post", "grad_res", "alpha")


def _gpu(host, c, dev, **kw):
    d = {k: torch.from_numpy(np.ascontiguousarray(host[k])).to(dev) for k in KEYS}
    gm, gb, ga = coeff.mhc_coeff_bwd(*(d[k] for k in KEYS), c, **kw)
    torch.cuda.synchronize()
    return gm.cpu().numpy(), gb.cpu().numpy(), ga.cpu().numpy()


def _oracle(host, c):
    n = host["pre"].shape[1]
    return cb.coeff_bwd(*(host[k] for k in KEYS), c, n)


def _check(host, c, dev, what, **kw):
    got = _gpu(host, c, dev, **kw)
    want = _oracle(host, c)
    for name, g, w in zip(("grad_mix", "grad_b", "grad_alpha"), got, want):
        assert_bytes_equal(g, w, f"{what} {name}")


@pytest.mark.parametrize("launches", [1, 2])
@pytest.mark.parametrize("n", [2, 4, 8])
@pytest.mark.parametrize("R", [1, 63, 64, 65, 300, 4096, 4097, 4161, 8257])
def test_bit_exact_against_the_oracle(device, n, R, launches):
    say(f"coeff bwd n={n} R={R} launches={launches}")
    _check(make_coeff_inputs(R, n, seed=R + n), 2.0, device, f"n={n} R={R}", launches=launches)


@pytest.mark.parametrize("R", [512, 2048, 8192])
def test_bit_exact_at_the_page_shapes(device, R):
    say(f"coeff bwd page shape R={R}")
    _check(make_coeff_inputs(R, 4, seed=0), 2.0, device, f"R={R}")


@pytest.mark.parametrize("c", [1.0, 3.0, 0.75, 2.0 ** 20])
def test_other_post_scales(device, c):
    say(f"coeff bwd post_scale={c}")
    _check(make_coeff_inputs(1000, 4, seed=3, post_scale=c), c, device, f"c={c}")


@pytest.mark.parametrize("launches", [1, 2])
@pytest.mark.parametrize("c", [3.0, 0.75, 7.0, 1.0 / 3.0, 5e-39, 1e30])
def test_post_quotient_is_correctly_rounded(device, c, launches):
    """Post values close to the scale, where s = post / c is near 1 and
    1 - s is exact, so an error of one unit in the last place of the
    quotient changes the derivative; plus post values down into the
    subnormal range. Non-power-of-two scales (and a subnormal one) make the
    quotient inexact. The kernel's division must give the oracle's
    correctly rounded quotient every time."""
    say(f"coeff bwd quotient c={c} launches={launches}")
    R, n = 4096, 8
    host = make_coeff_inputs(R, n, seed=77, post_scale=1.0)
    rng = np.random.default_rng(78)
    cf = np.float32(c)
    near = cf * (1.0 - rng.uniform(0.0, 2.0 ** -8, (R // 2, n)))
    wide = cf * np.exp2(-rng.uniform(0.0, 140.0, (R - R // 2, n)))
    host["post"] = np.ascontiguousarray(np.concatenate([near, wide]).astype(np.float32))
    host["grad_post"][:] = 1.0
    _check(host, float(cf), device, f"quotient c={c}", launches=launches)


@pytest.mark.parametrize("launches", [0, 1])
def test_large_batch(device, launches):
    """2^20 rows: 16,384 chunks, past the one-launch policy limit (the
    policy takes two launches); forced into one launch (its last block then
    walks 256 rounds of chunk sums) it must agree."""
    R = 1 << 20
    say(f"coeff bwd large R={R} launches={launches}")
    assert coeff.mhc_coeff_bwd_plan(R, 4, launches) == (2 if launches == 0 else 1)
    _check(make_coeff_inputs(R, 4, seed=11), 2.0, device, f"R={R}", launches=launches)


def _placed(R, n, col_vals):
    """Inputs whose derivative is zero except for residual column 0, which
    carries the given row values (d = grad_res there)."""
    h = make_coeff_inputs(R, n, seed=1)
    h["grad_pre"][:] = 0
    h["grad_post"][:] = 0
    h["grad_res"][:] = 0
    for r, v in col_vals.items():
        h["grad_res"][r, 0] = v
    return h


@pytest.mark.parametrize("launches", [1, 2])
@pytest.mark.parametrize("R,vals,want", [
    (4, {0: 1.0, 1: U, 3: U}, 1.0 + 2 * U),                      # first-stage tree
    (64, {0: 1.0, 32: U, 33: U}, 1.0),                            # 64-row chunks (not 32)
    (128, {0: 1.0, 64: U, 65: U}, 1.0 + 2 * U),                   # 64-row chunks (not 128)
    (65 * 64 + 1, {0: 1.0, 64: U, 65 * 64: U}, 1.0 + 2 * U),      # chunks strided over 64
    (128 * 64 + 1, {0: 1.0, 64 * 64: U, 128 * 64: U}, 1.0),       # ascending per accumulator
])
def test_row_order_hand_derived_cases(device, R, vals, want, launches):
    """The hand-derived values of the row order (derivations beside the same
    cases in tests/test_coeff_oracle.py), reached on the device."""
    say(f"coeff bwd row order R={R} launches={launches}")
    _, gb, _ = _gpu(_placed(R, 4, vals), 2.0, device, launches=launches)
    assert gb[8] == np.float32(want)
    assert np.all(gb[:8] == 0) and np.all(gb[9:] == 0)


def test_empty_batch_writes_zero_sums(device):
    say("coeff bwd R=0")
    d = {k: torch.empty((0,) + make_coeff_inputs(1, 4)[k].shape[1:], dtype=torch.float32,
                        device=device) for k in KEYS if k != "alpha"}
    alpha = torch.ones(3, device=device)
    gb = torch.full((24,), float("nan"), device=device)
    ga = torch.full((3,), float("nan"), device=device)
    gm, gb, ga = coeff.mhc_coeff_bwd(d["mix"], d["pre"], d["post"], d["grad_pre"],
                                     d["grad_post"], d["grad_res"], alpha, 2.0, grad_b=gb,
                                     grad_alpha=ga)
    torch.cuda.synchronize()
    assert gm.shape == (0, 24)
    assert gb.cpu().tolist() == [0.0] * 24 and ga.cpu().tolist() == [0.0] * 3
    assert not torch.signbit(gb).any()


def test_repeatable_and_independent_of_workspace_contents(device):
    """Twenty calls in each form on one workspace whose chunk-sum area is
    refilled with garbage before each call: identical bytes every time, and
    the arrival counter back at zero after every call."""
    say("coeff bwd repeat")
    host = make_coeff_inputs(5000, 4, seed=21)
    first = _gpu(host, 2.0, device)
    ws = torch.zeros(coeff.mhc_coeff_bwd_workspace_bytes(5000, 4), dtype=torch.uint8,
                     device=device)
    for k in range(40):
        ws[256:].fill_(0xFF if k % 2 else 0x7F)     # NaN patterns / large values
        got = _gpu(host, 2.0, device, workspace=ws, launches=1 + k % 2)
        for a, b, name in zip(got, first, ("grad_mix", "grad_b", "grad_alpha")):
            assert_bytes_equal(a, b, f"repeat {k} {name}")
        assert int(ws[:4].view(torch.int32).item()) == 0


@pytest.mark.parametrize("R", [4096, 8192])
def test_one_launch_form_sees_every_chunk_sum(device, R):
    """100 one-launch calls at 64 chunks (32 two-wave blocks arriving) and at
    128 chunks (32 four-wave blocks), each after the chunk-sum area was
    refilled with NaN patterns and each on fresh inputs: the last block must
    read every other block's sums, never a stale value (which would show as
    a NaN or a wrong sum)."""
    say(f"coeff bwd one-launch visibility R={R}")
    ws = torch.zeros(coeff.mhc_coeff_bwd_workspace_bytes(R, 4), dtype=torch.uint8,
                     device=device)
    keys = KEYS
    hosts = [make_coeff_inputs(R, 4, seed=100 + k) for k in range(4)]
    wants = [_oracle(h, 2.0) for h in hosts]
    devs = [[torch.from_numpy(h[k]).to(device) for k in keys] for h in hosts]
    for it in range(100):
        j = it % 4
        ws[256:].fill_(0xFF)
        gm, gb, ga = coeff.mhc_coeff_bwd(*devs[j], 2.0, workspace=ws, launches=1)
        torch.cuda.synchronize()
        assert_bytes_equal(gb.cpu().numpy(), wants[j][1], f"call {it} grad_b")
        assert_bytes_equal(ga.cpu().numpy(), wants[j][2], f"call {it} grad_alpha")
    assert int(ws[:4].view(torch.int32).item()) == 0


def test_calls_of_different_sizes_share_one_workspace(device):
    say("coeff bwd shared workspace")
    ws = torch.zeros(coeff.mhc_coeff_bwd_workspace_bytes(8192, 8), dtype=torch.uint8,
                     device=device)
    for R, n in ((8192, 8), (3, 4), (700, 2), (1, 8), (4096, 4)):
        _check(make_coeff_inputs(R, n, seed=R), 2.0, device, f"shared ws R={R} n={n}",
               workspace=ws)
        assert int(ws[:4].view(torch.int32).item()) == 0


def test_grad_mix_rows_do_not_depend_on_the_batch(device):
    say("coeff bwd row independence")
    host = make_coeff_inputs(700, 8, seed=5)
    whole = _gpu(host, 2.0, device)[0]
    parts = []
    for lo, hi in ((0, 1), (1, 129), (129, 700)):
        parts.append(_gpu({k: (v if k == "alpha" else v[lo:hi]) for k, v in host.items()},
                          2.0, device)[0])
    assert_bytes_equal(np.concatenate(parts), whole, "grad_mix split")


def test_special_values(device):
    say("coeff bwd special values")
    host = make_coeff_inputs(256, 4, seed=9)
    host["pre"][:8] = 0.0
    host["pre"][8:16] = 1.0
    host["post"][:8] = 2.0                      # post = c: saturated
    host["grad_pre"][16:24] = -0.0
    host["grad_post"][24:32] = np.float32(1e-39)  # denormal products
    host["grad_res"][32:40] = np.float32(3e-41)
    host["mix"][40:48] = np.float32(1e30)       # large products in the alpha terms
    host["grad_res"][48:56] = np.float32(3e38)  # overflow to +inf in grad_mix (alpha > 1)
    host["mix"][48:56] = np.float32(0.5)        # and in the sums, with one sign (no NaN)
    host["alpha"][2] = np.float32(1.25)
    _check(host, 2.0, device, "special")


@pytest.mark.parametrize("launches", [1, 2])
@pytest.mark.parametrize("shift", [1, 2, 3])
def test_buffers_aligned_to_4_bytes_only(device, shift, launches):
    """The header asks for 4-byte alignment only. Every tensor here starts
    `shift` floats past a 256-byte boundary (and the workspace 4 bytes
    past one), so no row starts on a 16-byte boundary; the bytes must be
    the oracle's."""
    say(f"coeff bwd shift={shift} launches={launches}")
    R, n = 1000, 4
    host = make_coeff_inputs(R, n, seed=60 + shift)

    def shifted(a):
        buf = torch.empty(a.size + shift + 64, dtype=torch.float32, device=device)
        t = buf[shift:shift + a.size].view(a.shape)
        t.copy_(torch.from_numpy(np.ascontiguousarray(a)).to(device))
        assert t.data_ptr() % 16 == 4 * shift
        return t

    d = {k: shifted(host[k]) for k in KEYS}
    gm = shifted(np.zeros((R, 24), np.float32))
    gb = shifted(np.zeros(24, np.float32))
    ga = shifted(np.zeros(3, np.float32))
    need = coeff.mhc_coeff_bwd_workspace_bytes(R, n)
    wbuf = torch.zeros(need + 64, dtype=torch.uint8, device=device)
    ws = wbuf[4:4 + need]
    coeff.mhc_coeff_bwd(*(d[k] for k in KEYS), 2.0, grad_mix=gm, grad_b=gb, grad_alpha=ga,
                        workspace=ws, launches=launches)
    torch.cuda.synchronize()
    want = _oracle(host, 2.0)
    for name, g, w in zip(("grad_mix", "grad_b", "grad_alpha"), (gm, gb, ga), want):
        assert_bytes_equal(g.cpu().numpy(), w, f"shift {shift} {name}")


def test_timed_call_records_both_events(device):
    say("coeff bwd timed")
    host = make_coeff_inputs(2048, 4, seed=2)
    ev = HipEvents(2)
    try:
        for launches in (1, 2):
            _gpu(host, 2.0, device, launches=launches, start_event=ev.h[0], stop_event=ev.h[1])
            ms = ev.elapsed_ms(0, 1)
            assert 0 < ms < 100
    finally:
        ev.close()


# ---------------------------------------------------------------------------
# 16-bit row tensors (mhc_coeff_bwd_ex through the binding's dtype dispatch)
# ---------------------------------------------------------------------------

TORCH16 = {"bf16": torch.bfloat16, "f16": torch.float16}


def _typed_host(R, n, seed, dtype, c=2.0):
    h = make_coeff_inputs(R, n, seed=seed, post_scale=c)
    return {k: (cb.narrow(v, dtype) if k != "alpha" else v) for k, v in h.items()}


def _gpu_typed(host, c, dev, dtype, **kw):
    d = {k: (torch.from_numpy(np.ascontiguousarray(host[k]).view(np.int16)).to(dev)
             .view(TORCH16[dtype]) if k != "alpha" else torch.from_numpy(host[k]).to(dev))
         for k in KEYS}
    gm, gb, ga = coeff.mhc_coeff_bwd(*(d[k] for k in KEYS), c, **kw)
    torch.cuda.synchronize()
    assert gm.dtype == TORCH16[dtype] and gb.dtype == torch.float32
    return gm.view(torch.int16).cpu().numpy().view(np.uint16), gb.cpu().numpy(), ga.cpu().numpy()


def _check_typed(host, c, dev, dtype, what, **kw):
    n = host["pre"].shape[1]
    got = _gpu_typed(host, c, dev, dtype, **kw)
    want = cb.coeff_bwd_typed(*(host[k] for k in KEYS), c, n, dtype)
    for name, g, w in zip(("grad_mix", "grad_b", "grad_alpha"), got, want):
        assert_bytes_equal(g, w, f"{what} {name}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("launches", [1, 2])
@pytest.mark.parametrize("n", [2, 4, 8])
@pytest.mark.parametrize("R", [1, 63, 65, 4097, 8257])
def test_typed_bit_exact_against_the_oracle(device, dtype, n, R, launches):
    say(f"coeff bwd {dtype} n={n} R={R} launches={launches}")
    _check_typed(_typed_host(R, n, R + n, dtype), 2.0, device, dtype, f"{dtype} n={n} R={R}",
                 launches=launches)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("R", [512, 2048, 8192])
def test_typed_page_shapes(device, dtype, R):
    say(f"coeff bwd {dtype} page shape R={R}")
    _check_typed(_typed_host(R, 4, 0, dtype), 2.0, device, dtype, f"{dtype} R={R}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("a2", [1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -8,
                                1.0 + 3 * 2.0 ** -8, 1.0003, 0.7, 3.0])
def test_typed_grad_mix_rounding(device, dtype, a2):
    """grad_mix = alpha * d on the residual columns with d = grad_res = +-2^k
    over the whole range of the format (and its largest values): with these
    gains the products are exact fp32 values on the format's ties (every
    binade, subnormals included) or just past its largest finite value, so
    the device's narrowing is checked at its decision points."""
    say(f"coeff bwd {dtype} grad_mix rounding alpha2={a2}")
    n, R = 4, 1024
    host = _typed_host(R, n, 5, dtype)
    lo, hi = (-24, 16) if dtype == "f16" else (-133, 128)
    k = np.arange(lo, hi)
    vals = np.concatenate([np.exp2(k), -np.exp2(k),
                           [65504.0, -65504.0, 65472.0] if dtype == "f16" else
                           [3.3895314e38, -3.3895314e38, 1.0]]).astype(np.float32)
    vals = np.resize(vals, R * n * n).reshape(R, n * n)
    host["grad_res"] = cb.narrow(vals, dtype)
    host["alpha"] = np.array([1.0, 1.0, a2], np.float32)
    _check_typed(host, 2.0, device, dtype, f"{dtype} rounding a2={a2}", launches=2)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_typed_buffers_aligned_to_2_bytes_only(device, dtype):
    """Row tensors and grad_mix one element past a 256-byte boundary (the
    16-bit forms need only 2-byte alignment)."""
    say(f"coeff bwd {dtype} 2-byte alignment")
    R, n = 1000, 4
    host = _typed_host(R, n, 61, dtype)

    def shifted(a, dt):
        buf = torch.empty(a.size + 64, dtype=dt, device=device)
        t = buf[1:1 + a.size].view(a.shape)
        t.copy_(torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(dt))
        assert t.data_ptr() % 4 == 2
        return t

    dt = TORCH16[dtype]
    d = {k: shifted(host[k], dt) for k in KEYS if k != "alpha"}
    alpha = torch.from_numpy(host["alpha"]).to(device)
    gm = shifted(np.zeros((R, 24), np.uint16), dt)
    got = coeff.mhc_coeff_bwd(*(d[k] for k in KEYS if k != "alpha"), alpha, 2.0, grad_mix=gm)
    torch.cuda.synchronize()
    want = cb.coeff_bwd_typed(*(host[k] for k in KEYS), 2.0, n, dtype)
    assert_bytes_equal(gm.view(torch.int16).cpu().numpy().view(np.uint16), want[0],
                       f"{dtype} shifted grad_mix")
    assert_bytes_equal(got[1].cpu().numpy(), want[1], f"{dtype} shifted grad_b")

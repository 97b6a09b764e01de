"""Pins of the coefficient-backward oracle (oracle/coeff_bwd.py).

The page ("perf: fuse mHC coefficient backward epilogue", Summary) names the
epilogue's parts but prints no formula, so the oracle cannot be compared with
values from the page; it is pinned here to what the mathematics fixes:

* the calculus of the reading: fp64 central differences of the forward being
  differentiated (sigmoid gates, affine z = alpha * mix + b) against the
  oracle's gradients, at every expansion rate and two post scales;
* hand-derived values: a one-row case worked out by hand in exact binary
  fractions, and discriminating inputs for every stage of the fixed row
  order (each expected value derived by hand from the order's definition,
  and each differing from what a plausible wrong order gives);
* special cases (alpha = 0, saturated gates, c = 1, one row) and the error
  bounds against correctly rounded fp64 sums.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import coeff_bwd as cb

U = 2.0 ** -24


def _inputs(R, n, seed, c=2.0):
    rng = np.random.default_rng(seed)
    m = cb.columns(n)
    f = lambda a: np.asarray(a, dtype=np.float32)
    return dict(mix=f(rng.standard_normal((R, m))), pre=f(rng.random((R, n))),
                post=f(rng.random((R, n)) * c), grad_pre=f(rng.standard_normal((R, n))),
                grad_post=f(rng.standard_normal((R, n))),
                grad_res=f(rng.standard_normal((R, n * n))),
                alpha=f(rng.uniform(0.5, 1.5, 3)))


def _run(d, c, n):
    return cb.coeff_bwd(d["mix"], d["pre"], d["post"], d["grad_pre"], d["grad_post"],
                        d["grad_res"], d["alpha"], c, n)


# ---------------------------------------------------------------------------
# Hand-computed case (exact binary fractions, every step exact)
# ---------------------------------------------------------------------------

def test_hand_case_one_row_n2():
    # n = 2: columns pre0 pre1 | post0 post1 | res00 res01 res10 res11; c = 2.
    # pre  = (1/2, 1/4), grad_pre  = (1, 2):
    #   d = 1 * (1/2 * 1/2) = 1/4,  2 * (1/4 * 3/4) = 3/8
    # post = (1, 1/2) -> s = post / 2 = (1/2, 1/4), grad_post = (1, -1):
    #   d = 1 * (1 * 1/2) = 1/2,   -1 * (1/2 * 3/4) = -3/8
    # res: d = grad_res = (1, 2, 3, 4)
    # alpha = (2, 1/2, 1): grad_mix = (1/2, 3/4, 1/4, -3/16, 1, 2, 3, 4)
    # one row: grad_b = d
    # mix = (1..8): alpha grads: pre 1/4*1 + 3/8*2 = 1; post 1/2*3 - 3/8*4 = 0;
    #   res 1*5 + 2*6 + 3*7 + 4*8 = 70
    f = lambda *v: np.array([v], dtype=np.float32)
    gm, gb, ga = cb.coeff_bwd(f(1, 2, 3, 4, 5, 6, 7, 8), f(0.5, 0.25), f(1.0, 0.5), f(1, 2),
                              f(1, -1), f(1, 2, 3, 4), np.array([2, 0.5, 1], np.float32), 2.0, 2)
    assert gm.tolist() == [[0.5, 0.75, 0.25, -0.1875, 1, 2, 3, 4]]
    assert gb.tolist() == [0.25, 0.375, 0.5, -0.375, 1, 2, 3, 4]
    assert ga.tolist() == [1.0, 0.0, 70.0]


def test_group_sums_run_over_columns_in_ascending_order():
    """e[r, k] adds d * mix over the group's columns in ascending order from
    +0.0. One row, n = 2, only the residual group non-zero, mix = 1 and
    grad_res = (1, -1, 2^-25, 0): ascending, ((1 + (-1)) + 2^-25) = 2^-25;
    descending, 2^-25 + (-1) ties to -1 (even), and -1 + 1 = 0. With one row
    the row sum of e is e itself, so grad_alpha[2] = 2^-25."""
    f = lambda *v: np.array([v], dtype=np.float32)
    tiny = 2.0 ** -25
    _, _, ga = cb.coeff_bwd(f(0, 0, 0, 0, 1, 1, 1, 1), f(0.5, 0.5), f(1.0, 1.0), f(0, 0), f(0, 0),
                            f(1.0, -1.0, tiny, 0.0), np.array([1, 1, 1], np.float32), 2.0, 2)
    assert ga.tolist() == [0.0, 0.0, tiny]


# ---------------------------------------------------------------------------
# The fixed row order: hand-derived discriminators
# ---------------------------------------------------------------------------

def _col(R, vals):
    x = np.zeros((R, 1), dtype=np.float32)
    for r, v in vals.items():
        x[r, 0] = v
    return x


def test_row_sum_first_stage_is_the_halving_tree():
    # rows 0..3 = 1, 2^-24, 0, 2^-24. Tree: offset 2 gives x1 = 2^-24 + 2^-24
    # = 2^-23 and x0 = 1; offset 1 gives 1 + 2^-23 (exact). A sequential sum
    # rounds 1 + 2^-24 to 1 (tie to even) twice and gives 1.
    got = cb.row_sum(_col(4, {0: 1.0, 1: U, 3: U}))
    assert got[0] == np.float32(1.0 + 2 * U)


def test_row_sum_chunks_are_64_rows():
    # rows 0 = 1, 32 = 33 = 2^-24, one chunk of 64: offset 32 adds row 32 to
    # row 0 (1 + 2^-24 -> 1) and row 33 to row 1; offset 1 adds 2^-24 to 1
    # again -> 1. With 32-row chunks the second chunk would sum to 2^-23 and
    # the result would be 1 + 2^-23.
    assert cb.row_sum(_col(64, {0: 1.0, 32: U, 33: U}))[0] == np.float32(1.0)
    # rows 0 = 1, 64 = 65 = 2^-24: chunk 1 sums to 2^-23 (offset 1), stage 2
    # adds it to chunk 0's 1 -> 1 + 2^-23. One 128-row tree would give 1.
    assert cb.row_sum(_col(128, {0: 1.0, 64: U, 65: U}))[0] == np.float32(1.0 + 2 * U)


def test_row_sum_second_stage_strides_chunks_over_64_accumulators():
    # 66 chunks. Chunk sums: P0 = 1, P1 = 2^-24, P65 = 2^-24. Accumulator 1
    # gets P1 and P65 (65 mod 64 = 1): 2^-23; the final tree adds it to
    # accumulator 0's 1 -> 1 + 2^-23. Visiting the chunk sums one after
    # another would give 1; giving each accumulator a contiguous run of chunks
    # (0-1 to the first, ...) would also give 1.
    R = 65 * 64 + 1
    assert cb.row_sum(_col(R, {0: 1.0, 64: U, 65 * 64: U}))[0] == np.float32(1.0 + 2 * U)
    # 129 chunks: P0 = 1, P64 = 2^-24, P128 = 2^-24 all go to accumulator 0,
    # in ascending order: (1 + 2^-24) + 2^-24 rounds to 1 twice.
    R = 128 * 64 + 1
    assert cb.row_sum(_col(R, {0: 1.0, 64 * 64: U, 128 * 64: U}))[0] == np.float32(1.0)


def test_row_sum_empty_and_single():
    assert cb.row_sum(np.zeros((0, 3), np.float32)).tolist() == [0.0, 0.0, 0.0]
    x = np.array([[3.5, -2.0, -0.0]], np.float32)
    got = cb.row_sum(x)
    assert got.tolist() == [3.5, -2.0, 0.0]
    assert not np.signbit(got[2])        # -0 + (+0) is +0


@pytest.mark.parametrize("R", [1, 63, 64, 65, 1000, 4097, 9000])
def test_row_sum_within_error_bound_of_exact_sum(R):
    rng = np.random.default_rng(R)
    x = rng.standard_normal((R, 5)).astype(np.float32) * np.float32(3.0)
    got = cb.row_sum(x)
    for v in range(5):
        exact = math.fsum(x[:, v].astype(np.float64))
        mag = math.fsum(np.abs(x[:, v]).astype(np.float64))
        assert abs(float(got[v]) - exact) <= cb.reduction_error_bound(R) * mag, v


# ---------------------------------------------------------------------------
# Calculus: the gradients of the forward being differentiated
# ---------------------------------------------------------------------------

def _loss64(mix, b, alpha, gp, gq, gr, c, n):
    k = cb.groups(n)
    z = alpha[k][None, :] * mix + b[None, :]
    sig = 1.0 / (1.0 + np.exp(-z))
    return (math.fsum((gp * sig[:, :n]).ravel()) + math.fsum((gq * c * sig[:, n:2 * n]).ravel())
            + math.fsum((gr * z[:, 2 * n:]).ravel()))


@pytest.mark.parametrize("n", [2, 4, 8])
@pytest.mark.parametrize("c", [1.0, 2.0, 3.0])
def test_gradients_match_finite_differences_of_the_forward(n, c):
    R, m = 5, cb.columns(n)
    rng = np.random.default_rng(100 + n)
    mix = rng.standard_normal((R, m))
    b = rng.standard_normal(m) * 0.5
    alpha = rng.uniform(0.5, 1.5, 3)
    gp, gq, gr = (rng.standard_normal((R, n)), rng.standard_normal((R, n)),
                  rng.standard_normal((R, n * n)))
    # the saved activations the epilogue receives
    k = cb.groups(n)
    z = alpha[k][None, :] * mix + b[None, :]
    sig = 1.0 / (1.0 + np.exp(-z))
    f = lambda a: np.asarray(a, dtype=np.float32)
    gm, gb, ga = cb.coeff_bwd(f(mix), f(sig[:, :n]), f(c * sig[:, n:2 * n]), f(gp), f(gq), f(gr),
                              f(alpha), c, n)
    L = lambda mx, bb, al: _loss64(mx, bb, al, gp, gq, gr, c, n)
    h = 1e-6

    def fd(vec, idx, fn):
        a, bm = vec.copy(), vec.copy()
        a[idx] += h
        bm[idx] -= h
        return (fn(a) - fn(bm)) / (2 * h)

    # inputs were rounded to fp32 for the oracle: compare at ~1e-5
    tol = lambda want: 2e-5 * (abs(want) + 1.0)
    for r in range(R):
        for j in range(m):
            want = fd(mix, (r, j), lambda x: L(x, b, alpha))
            assert abs(gm[r, j] - want) <= tol(want), ("grad_mix", r, j, gm[r, j], want)
    for j in range(m):
        want = fd(b, j, lambda x: L(mix, x, alpha))
        assert abs(gb[j] - want) <= tol(want) * R, ("grad_b", j, gb[j], want)
    for g in range(3):
        want = fd(alpha, g, lambda x: L(mix, b, x))
        assert abs(ga[g] - want) <= tol(want) * R * m, ("grad_alpha", g, ga[g], want)


# ---------------------------------------------------------------------------
# Special cases and error bounds
# ---------------------------------------------------------------------------

def test_zero_alpha_zeroes_grad_mix_only():
    d = _inputs(70, 4, 1)
    d["alpha"] = np.zeros(3, np.float32)
    gm, gb, ga = _run(d, 2.0, 4)
    assert np.all(gm == 0)
    assert np.any(gb != 0) and np.all(ga != 0)


def test_saturated_gates_have_zero_derivative():
    d = _inputs(8, 4, 2)
    d["pre"][:4] = 0.0
    d["pre"][4:] = 1.0
    d["post"][:4] = 0.0
    d["post"][4:] = 2.0          # post = c: sigmoid saturated at 1
    gm, gb, _ = _run(d, 2.0, 4)
    assert np.all(gm[:, :8] == 0) and np.all(gb[:8] == 0)


def test_unit_post_scale_makes_post_like_pre():
    d = _inputs(33, 4, 3, c=1.0)
    d["post"] = d["pre"].copy()
    d["grad_post"] = d["grad_pre"].copy()
    d["alpha"][1] = d["alpha"][0]
    gm, gb, _ = _run(d, 1.0, 4)
    assert np.array_equal(gm[:, :4], gm[:, 4:8]) and np.array_equal(gb[:4], gb[4:8])


def _rn32(x) -> float:
    """Exact rational -> nearest fp32 (ties to even), for positive normal x."""
    from fractions import Fraction as Fr
    x = Fr(x)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fr(2) ** e > x:
        e -= 1
    y = x * Fr(2) ** (23 - e)                 # in [2^23, 2^24)
    fl = y.numerator // y.denominator
    rem = y - fl
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and fl % 2 == 1):
        fl += 1
    return float(Fr(fl) * Fr(2) ** (e - 23))


def test_post_gate_divides_by_the_scale():
    # c = 3: the sigmoid is s = rn(q / 3), one correctly rounded division. A
    # reciprocal form rn(q * rn(1/3)) is a plausible shortcut that differs
    # from it; find the first post value from 1.5 upward where
    # d = rn(q * rn(1 - s)) differs between the two, in exact rational
    # arithmetic (1 - s is exact for s in [1/2, 1]), and check that the oracle
    # follows the division.
    from fractions import Fraction as Fr
    ic = Fr(_rn32(Fr(1, 3)))
    assert ic == Fr(11184811, 2 ** 25)
    q = np.float32(1.5)
    for _ in range(100000):
        Q = Fr(float(q))
        want = _rn32(Q * (1 - Fr(_rn32(Q / 3))))
        other = _rn32(Q * (1 - Fr(_rn32(Q * ic))))
        if want != other:
            break
        q = np.nextafter(q, np.float32(3.0))
    else:
        raise AssertionError("no discriminating value found")
    d = _inputs(1, 2, 8)
    d["post"][0] = [q, q]
    d["grad_post"][0] = [1.0, -1.0]
    dz = cb.dz(d["pre"], d["post"], d["grad_pre"], d["grad_post"], d["grad_res"], 3.0)
    assert dz[0, 2] == np.float32(want) and dz[0, 3] == np.float32(-want)


@pytest.mark.parametrize("c", [3.0, 0.75, 7.0, 1.0 / 3.0])
def test_post_sigmoid_is_the_correctly_rounded_quotient(c):
    """s = post / c is the fp32 value nearest the exact quotient, for
    non-power-of-two scales, checked in exact rational arithmetic on the
    quantity the post derivative is built from (1 - s, exact for s in
    [1/2, 1])."""
    from fractions import Fraction as Fr
    rng = np.random.default_rng(11)
    cf = np.float32(c)
    C = Fr(float(cf))
    post = (cf * rng.uniform(0.5, 1.0, 64)).astype(np.float32)
    d = _inputs(64, 2, 9)
    d["post"][:, 0] = post
    d["post"][:, 1] = post
    d["grad_post"][:] = 1.0
    dz = cb.dz(d["pre"], d["post"], d["grad_pre"], d["grad_post"], d["grad_res"], float(cf))
    for r, q in enumerate(post):
        Q = Fr(float(q))
        s = Fr(_rn32(Q / C))
        if not (Fr(1, 2) <= s <= 1):
            continue
        want = _rn32(Q * (1 - s)) if s < 1 else 0.0
        assert dz[r, 2] == np.float32(want), (c, float(q))


def test_one_row_grad_b_is_the_row_derivative():
    d = _inputs(1, 8, 4)
    gm, gb, _ = _run(d, 2.0, 8)
    dz = cb.dz(d["pre"], d["post"], d["grad_pre"], d["grad_post"], d["grad_res"], 2.0)
    assert np.array_equal(gb, dz[0])


@pytest.mark.parametrize("c", [2.0, 3.0, 0.75])
@pytest.mark.parametrize("n,R", [(2, 300), (4, 2048), (8, 257)])
def test_within_error_bounds_of_fp64(n, R, c):
    d = _inputs(R, n, 5 + n, c)
    gm, gb, ga = _run(d, c, n)
    ex = cb.coeff_bwd_exact(d["mix"], d["pre"], d["post"], d["grad_pre"], d["grad_post"],
                            d["grad_res"], d["alpha"], c, n)
    k = cb.groups(n)
    al = np.abs(d["alpha"].astype(np.float64))[k][None, :]
    assert np.all(np.abs(gm - ex["grad_mix"]) <= 6 * U * al * ex["mag_d"] + 1e-44)
    rb = cb.reduction_error_bound(R)
    assert np.all(np.abs(gb - ex["grad_b"]) <= (rb + 5 * U) * ex["mag_b"] * 1.01)
    width = max(n, n * n)
    ra = cb.reduction_error_bound(R, width)
    assert np.all(np.abs(ga - ex["grad_alpha"]) <= (ra + 6 * U) * ex["mag_alpha"] * 1.01)


def test_empty_batch_gives_zero_sums():
    d = _inputs(0, 4, 6)
    gm, gb, ga = _run(d, 2.0, 4)
    assert gm.shape == (0, 24) and gb.tolist() == [0.0] * 24 and ga.tolist() == [0.0] * 3


def test_argument_checks():
    d = _inputs(4, 4, 7)
    with pytest.raises(ValueError):
        cb.coeff_bwd(d["mix"], d["pre"], d["post"], d["grad_pre"], d["grad_post"],
                     d["grad_res"], d["alpha"], 2.0, 3)
    with pytest.raises(ValueError):
        cb.coeff_bwd(d["mix"][:, :20], d["pre"], d["post"], d["grad_pre"], d["grad_post"],
                     d["grad_res"], d["alpha"], 2.0, 4)
    with pytest.raises(ValueError):
        cb.coeff_bwd(d["mix"].astype(np.float64), d["pre"], d["post"], d["grad_pre"],
                     d["grad_post"], d["grad_res"], d["alpha"], 2.0, 4)


# ---------------------------------------------------------------------------
# 16-bit inputs (bf16 / fp16 row tensors; grad_mix in the input's format)
# ---------------------------------------------------------------------------

def _f16_nearest(x: float) -> float:
    """Independent round-to-nearest-even of a finite float to IEEE binary16,
    by integer rounding of x / quantum in float64 (exact: the quotient is a
    power-of-two scaling; Python's round() breaks ties to even)."""
    a = abs(x)
    if a == 0.0:
        return x
    m, e = math.frexp(a)                      # a = m 2^e, m in [0.5, 1)
    quantum = 2.0 ** max(e - 11, -24)         # 11 significant bits; subnormal spacing 2^-24
    r = round(a / quantum) * quantum
    if r > 65504.0:                          # 65520 and up round past the largest finite
        r = math.inf
    return math.copysign(r, x)


def _f16_decode(b: int) -> float:
    """binary16 bit pattern -> value, from the format's definition."""
    s, e, f = b >> 15, (b >> 10) & 0x1F, b & 0x3FF
    if e == 0x1F:
        return math.nan if f else math.copysign(math.inf, -1.0 if s else 1.0)
    v = (f / 1024.0) * 2.0 ** -14 if e == 0 else (1.0 + f / 1024.0) * 2.0 ** (e - 15)
    return -v if s else v


def test_f16_widening_is_exact_on_every_pattern():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = cb.widen(b, "f16").astype(np.float64)
    want = np.array([_f16_decode(int(v)) for v in b])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_f16_narrowing_matches_an_independent_rounding():
    """Hand ties and overflow, then every fp32 binade from 2^-27 to 2^16:
    random patterns plus each binade's exact ties and their neighbours."""
    hand = {1.0 + 2.0 ** -11: 0x3C00, 1.0 + 3 * 2.0 ** -11: 0x3C02, 65504.0: 0x7BFF,
            65519.996: 0x7BFF, 65520.0: 0x7C00, 2.0 ** -24: 0x0001, 2.0 ** -25: 0x0000,
            3 * 2.0 ** -26: 0x0001, -2.0 ** -14: 0x8400, 1e-9: 0x0000}
    for x, bits in hand.items():
        assert int(cb.narrow(np.array([x], np.float32), "f16")[0]) == bits, x
    rng = np.random.default_rng(16)
    pats = []
    for e in range(-27 + 127, 17 + 127):
        base = np.uint32(e) << np.uint32(23)
        mant = rng.integers(0, 1 << 23, 600, dtype=np.uint32)
        ties = (np.arange(0, 1 << 10, dtype=np.uint32) << np.uint32(13)) | np.uint32(0x1000)
        pats += [base | mant, base | ties, base | (ties + 1), base | (ties - 1)]
    p = np.concatenate(pats)
    p = np.concatenate([p, p | np.uint32(0x80000000)])
    x = p.view(np.float32)
    got = cb.widen(cb.narrow(x, "f16"), "f16").astype(np.float64)
    want = np.array([_f16_nearest(float(v)) for v in x])
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_bf16_and_f32_formats_round_trip():
    x = np.array([1.0, -2.5, 3e38, 1e-40], np.float32)
    assert np.array_equal(cb.narrow(x, "f32"), x) and cb.widen(x, "f32") is x
    b = cb.narrow(x, "bf16")
    assert b.dtype == np.uint16 and np.array_equal(cb.widen(b, "bf16")[:2], x[:2])
    with pytest.raises(ValueError):
        cb.widen(x, "f16")
    with pytest.raises(ValueError):
        cb.narrow(x, "f8")


def _typed_inputs(R, n, seed, dtype, c=2.0):
    d = _inputs(R, n, seed, c)
    return {k: (cb.narrow(v, dtype) if k != "alpha" else v) for k, v in d.items()}


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_typed_hand_case_one_row_n2(dtype):
    # The fp32 hand case's inputs and results are exact in both 16-bit
    # formats, so the typed epilogue gives the same values.
    f = lambda v: cb.narrow(np.array([v], np.float32), dtype)
    mix = f([1, 2, 3, 4, 5, 6, 7, 8])
    pre, post = f([0.5, 0.25]), f([1.0, 0.5])
    gp, gq, gr = f([1, 2]), f([1, -1]), f([1, 2, 3, 4])
    alpha = np.array([2.0, 0.5, 1.0], np.float32)
    gm, gb, ga = cb.coeff_bwd_typed(mix, pre, post, gp, gq, gr, alpha, 2.0, 2, dtype)
    assert gm.dtype == np.uint16 and gb.dtype == np.float32 and ga.dtype == np.float32
    assert cb.widen(gm, dtype)[0].tolist() == [0.5, 0.75, 0.25, -0.1875, 1, 2, 3, 4]
    assert gb.tolist() == [0.25, 0.375, 0.5, -0.375, 1, 2, 3, 4]
    assert ga.tolist() == [1.0, 0.0, 70.0]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("n,R", [(2, 300), (4, 2048), (8, 257)])
def test_typed_within_error_bounds_of_fp64(dtype, n, R):
    """grad_mix within half an ulp of the 16-bit format plus the fp32
    evaluation error; the fp32 sums within the fp32 bounds: the sums are
    taken from the fp32 derivatives, never from the rounded grad_mix."""
    d = _typed_inputs(R, n, 30 + n, dtype)
    gm, gb, ga = cb.coeff_bwd_typed(*(d[k] for k in cb.ROW_INPUTS), d["alpha"], 2.0, n, dtype)
    w = {k: cb.widen(d[k], dtype) for k in cb.ROW_INPUTS}
    ex = cb.coeff_bwd_exact(*(w[k] for k in cb.ROW_INPUTS), d["alpha"], 2.0, n)
    k = cb.groups(n)
    al = np.abs(d["alpha"].astype(np.float64))[k][None, :]
    got = cb.widen(gm, dtype).astype(np.float64)
    bits = 8 if dtype == "bf16" else 11
    half_ulp = np.ldexp(1.0, np.frexp(np.abs(got))[1] - bits - 1)
    half_ulp = np.maximum(half_ulp, 2.0 ** -134 if dtype == "bf16" else 2.0 ** -25)
    assert np.all(np.abs(got - ex["grad_mix"]) <= half_ulp * 1.0001 + 6 * U * al * ex["mag_d"]
                  + 1e-44)
    rb = cb.reduction_error_bound(R)
    assert np.all(np.abs(gb - ex["grad_b"]) <= (rb + 5 * U) * ex["mag_b"] * 1.01)
    ra = cb.reduction_error_bound(R, max(n, n * n))
    assert np.all(np.abs(ga - ex["grad_alpha"]) <= (ra + 6 * U) * ex["mag_alpha"] * 1.01)


def test_typed_f32_is_the_plain_epilogue():
    d = _inputs(70, 4, 12)
    a = cb.coeff_bwd_typed(*(d[k] for k in cb.ROW_INPUTS), d["alpha"], 2.0, 4, "f32")
    b = _run(d, 2.0, 4)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))

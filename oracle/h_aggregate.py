"""Plain CPU oracle for the mHC pre / H-aggregate operation and its backward.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline use it. It shares no code, header, helper, table or constant
generator with the HIP path.

Sources (the pages this repository works from):

* "Add batch-invariant h_aggregate kernel" (RL-Kernel pull request 366),
  section *Summary*: the shapes residual[T,4,H] bf16, pre[T,4] fp32,
  output[T,H] bf16, and the formula
  out = bf16((pre0*r0 + pre1*r1) + (pre2*r2 + pre3*r3)).
* Same page, section *Batch invariance*: fp32 multiplies and adds each
  rounded to nearest (no fused multiply-add), the fixed (0+1)+(2+3) addition
  tree, and bf16 conversion only where data enters (exact widening) and
  leaves (one rounding).
* Same page, the maintainer's review comment: a backward is asked for so that
  training can converge. Its formulas are the derivative of the forward
  formula: d out / d r_i = pre_i and d out / d pre_i = r_i, so
  grad_residual[t,i,h] = pre[t,i] * grad_out[t,h] (rounded once to bf16) and
  grad_pre[t,i] = sum over h of grad_out[t,h] * residual[t,i,h] (kept fp32).

Readings taken where the pages are silent (each is listed in the design
notes of this repository):

* Expansion rates 2 and 8 (the second page's sibling implementation covers
  HC in {2, 4, 8}; the first page fixes 4): the forward's association is the
  balanced pairwise tree that reduces to (0+1)+(2+3) at 4; the backward is
  per stream and needs no change.

* fp32 rounding is round-to-nearest-even; bf16 rounding is
  round-to-nearest-even; denormals are kept (gradual underflow).
* NaN: the bf16 result of a NaN is a quiet NaN; only "is NaN" is specified.
* The order of the grad_pre sum over H is this repository's own fixed tree,
  `canonical_tree_sum` below. Any fixed order satisfies the request for a
  deterministic backward; this one is the contract both sides implement.

Arithmetic model: every fp32 operation is one numpy float32 ufunc call
(np.multiply / np.add on float32 arrays), which is IEEE round-to-nearest-even
per element with no contraction. Loops run over the reduction order exactly as
defined; numpy only vectorises across independent tokens / streams. No
np.sum, np.dot, einsum or similar call appears in an fp32 path, since those
impose their own association.

Pins: every function here is checked in tests/test_oracle.py against values
fixed by hand derivation, exact fp64/rational arithmetic, closed forms and
invariants (see that file for the list).
"""

from __future__ import annotations

import numpy as np

# Hyper-connection expansion rate: the residual stream holds 4 copies
# ("Add batch-invariant h_aggregate kernel", Summary: residual [T, 4, H]).
HC = 4

# Constants of this repository's fixed grad_pre reduction order (see
# canonical_tree_sum): 8 consecutive hidden elements form a group, groups are
# dealt round-robin to 256 accumulator lanes, which form 4 waves of 64.
GROUP = 8
LANES = 256
WAVE = 64
WAVES = LANES // WAVE


# ---------------------------------------------------------------------------
# Conversions ("Batch invariance": bf16 conversion only at the boundaries)
# ---------------------------------------------------------------------------

def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 values, exactly.

    A bf16 number is the top half of the fp32 number with the same value, so
    the widening is a 16-bit left shift of the bit pattern. No rounding.
    """
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("widen_bf16 expects uint16 bit patterns")
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """float32 values -> bf16 bit patterns (uint16), round to nearest even.

    Dropping the low 16 bits of the fp32 pattern truncates toward zero in
    magnitude. Adding 0x7FFF plus the lowest kept bit before the shift rounds
    to nearest with ties to the even kept pattern; a carry out of the
    mantissa moves into the exponent, which is the correct next binade, and
    the largest finite values carry into the infinity pattern (overflow to
    Inf). Subnormals follow the same rule because bf16 and fp32 share the
    exponent field. Infinities pass through unchanged. NaN inputs give a
    quiet NaN with the sign and top payload bits kept.
    """
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError("bf16_rne expects float32 input")
    u = x.view(np.uint32).astype(np.uint64)
    kept_lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = (u + np.uint64(0x7FFF) + kept_lsb) >> np.uint64(16)
    is_nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    quiet = (u >> np.uint64(16)) | np.uint64(0x0040)
    return np.where(is_nan, quiet, rounded).astype(np.uint16)


# ---------------------------------------------------------------------------
# Forward ("Add batch-invariant h_aggregate kernel", Summary and
# Batch invariance)
# ---------------------------------------------------------------------------

# Expansion rates this oracle evaluates: the page's 4, and 2 and 8 (the
# sibling implementation of the second page covers HC in {2, 4, 8}).
SUPPORTED_HC = (2, 4, 8)


def _check_fwd_args(residual: np.ndarray, pre: np.ndarray, n: int | None = HC
                    ) -> tuple[int, int]:
    """Shapes [T, n, H] / [T, n]; n=None accepts any supported expansion."""
    if residual.dtype != np.uint16 or residual.ndim != 3:
        raise ValueError("residual must be uint16 bf16 bits of shape [T, n, H]")
    got_n = residual.shape[1]
    if (n is not None and got_n != n) or got_n not in SUPPORTED_HC:
        raise ValueError(f"residual has {got_n} streams; expected {n if n else SUPPORTED_HC}")
    if pre.dtype != np.float32 or pre.shape != (residual.shape[0], got_n):
        raise ValueError("pre must be float32 of shape [T, n]")
    return residual.shape[0], residual.shape[2]


def pairwise_tree(p: list[np.ndarray]) -> np.ndarray:
    """Balanced pairwise fp32 sum of 2, 4 or 8 arrays: adjacent pairs first,
    then pairs of pairs. For 4 terms this is the page's (0+1)+(2+3); for 8 it
    is ((0+1)+(2+3))+((4+5)+(6+7)); for 2 it is 0+1."""
    level = list(p)
    while len(level) > 1:
        with np.errstate(over="ignore", invalid="ignore"):
            level = [np.add(level[2 * j], level[2 * j + 1]) for j in range(len(level) // 2)]
    return level[0]


def h_aggregate_fwd(residual: np.ndarray, pre: np.ndarray) -> np.ndarray:
    """out[t,h] = bf16( (pre0*r0 + pre1*r1) + (pre2*r2 + pre3*r3) ).

    residual: uint16 [T,4,H] (bf16 bits); pre: float32 [T,4].
    Returns uint16 [T,H] (bf16 bits).

    Each product and each sum is one fp32 round-to-nearest operation; the
    association is the fixed tree (0+1)+(2+3); the result is rounded to bf16
    once.
    """
    T, H = _check_fwd_args(residual, pre)
    r = widen_bf16(residual)                                   # [T,4,H] fp32, exact
    with np.errstate(over="ignore", invalid="ignore"):         # Inf / NaN are IEEE results
        p = [np.multiply(pre[:, i:i + 1], r[:, i, :]) for i in range(HC)]
        s01 = np.add(p[0], p[1])
        s23 = np.add(p[2], p[3])
        y = np.add(s01, s23)
    assert y.dtype == np.float32 and y.shape == (T, H)
    return bf16_rne(y)


def h_aggregate_fwd_n(residual: np.ndarray, pre: np.ndarray) -> np.ndarray:
    """Forward for any supported expansion n (residual [T,n,H], pre [T,n]):
    out = bf16( pairwise_tree(pre_i * r_i) ). For n = 4 it is exactly
    h_aggregate_fwd (the page's formula); n = 2 and 8 generalise its
    association as a balanced pairwise tree."""
    T, H = _check_fwd_args(residual, pre, None)
    n = residual.shape[1]
    r = widen_bf16(residual)
    with np.errstate(over="ignore", invalid="ignore"):
        p = [np.multiply(pre[:, i:i + 1], r[:, i, :]) for i in range(n)]
    y = pairwise_tree(p)
    assert y.dtype == np.float32 and y.shape == (T, H)
    return bf16_rne(y)


def h_aggregate_fwd_exact(residual: np.ndarray, pre: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """fp64 value of sum_i pre_i * r_i, and of sum_i |pre_i * r_i| (any
    supported n).

    Used only to check the fp32 oracle. Every product of an fp32 and a bf16
    number has at most 24 + 8 significant bits and is exact in fp64; the
    n-1 fp64 additions add a relative error of at most (n-1) * 2**-53 of
    sum |pre_i * r_i|, far below a bf16 ulp.
    """
    _check_fwd_args(residual, pre, None)
    r = widen_bf16(residual).astype(np.float64)
    pw = pre.astype(np.float64)[:, :, None]
    prod = pw * r                                              # exact
    exact = np.zeros(prod.shape[0:1] + prod.shape[2:], np.float64)
    mag = np.zeros_like(exact)
    for i in range(prod.shape[1]):
        exact = exact + prod[:, i]
        mag = mag + np.abs(prod[:, i])
    return exact, mag


# ---------------------------------------------------------------------------
# Backward (requested in the review comments of "Add batch-invariant
# h_aggregate kernel"; formulas are the derivative of the Summary formula)
# ---------------------------------------------------------------------------

def _check_bwd_args(residual, pre, grad_out) -> tuple[int, int]:
    T, H = _check_fwd_args(residual, pre, None)
    if grad_out.dtype != np.uint16 or grad_out.shape != (T, H):
        raise ValueError("grad_out must be uint16 bf16 bits of shape [T, H]")
    return T, H


def grad_residual_ref(pre: np.ndarray, grad_out: np.ndarray) -> np.ndarray:
    """grad_residual[t,i,h] = bf16( pre[t,i] * grad_out[t,h] ), one fp32 product.

    pre: float32 [T,n]; grad_out: uint16 [T,H]. Returns uint16 [T,n,H].
    The gradient is written, not accumulated into an existing buffer.
    """
    g = widen_bf16(grad_out)                                   # [T,H]
    with np.errstate(over="ignore"):
        prod = np.multiply(pre[:, :, None], g[:, None, :])    # [T,4,H] fp32 RN
    return bf16_rne(prod)


def grad_residual_acc_ref(pre: np.ndarray, grad_out: np.ndarray,
                          grad_residual_in: np.ndarray) -> np.ndarray:
    """Accumulating form: grad_residual[t,i,h] += pre[t,i] * grad_out[t,h].

    Reading taken (the pages only ask for a backward): the existing bf16
    value is widened exactly, the fp32 product pre*g (one rounding) is added
    to it in fp32 (one rounding), and the sum is rounded to bf16 once.
    grad_residual_in: uint16 [T,4,H]. Returns the updated uint16 [T,4,H].
    """
    g = widen_bf16(grad_out)
    old = widen_bf16(grad_residual_in)
    with np.errstate(over="ignore", invalid="ignore"):
        prod = np.multiply(pre[:, :, None], g[:, None, :])    # [T,4,H] fp32 RN
        total = np.add(old, prod)                              # fp32 RN
    return bf16_rne(total)


def grad_pre_products(residual: np.ndarray, grad_out: np.ndarray) -> np.ndarray:
    """q[t,i,h] = grad_out[t,h] * residual[t,i,h] in fp32.

    Both factors are bf16 (8 significant bits each), so the product has at
    most 16 significant bits and the fp32 multiply is exact whenever the
    product lies in fp32's normal range. Products below 2**-126 fall into the
    subnormal range, where fewer bits are available, and are rounded to
    nearest like any other fp32 product; products above the largest finite
    fp32 overflow. The function asserts exactness against fp64 for the
    products in the normal range.
    """
    g = widen_bf16(grad_out)
    r = widen_bf16(residual)
    with np.errstate(over="ignore"):
        q = np.multiply(g[:, None, :], r)
    q64 = g.astype(np.float64)[:, None, :] * r.astype(np.float64)
    a64 = np.abs(q64)
    normal = (a64 >= np.finfo(np.float32).tiny) & (a64 <= np.finfo(np.float32).max)
    assert np.array_equal(q.astype(np.float64)[normal], q64[normal]), \
        "bf16 x bf16 product in the normal range not exact in fp32"
    return q


def canonical_tree_sum(q: np.ndarray) -> np.ndarray:
    """Fixed-order fp32 sum over the last axis (length H) of q.

    This repository's reduction order for grad_pre. It depends only on H, so
    the result for one token never depends on how many other tokens are in
    the batch or how they are partitioned.

    1. 256 accumulator lanes start at +0.0.
    2. The hidden axis is cut into groups of 8 consecutive elements
       (group k holds h = 8k .. 8k+7; the last group may be short). Groups
       are visited in ascending k; group k belongs to lane k mod 256, and its
       elements are added to that lane's accumulator one at a time in
       ascending h, each addition rounded to fp32.
    3. The lanes form 4 waves of 64 (wave w = lanes 64w .. 64w+63). Within a
       wave, with x[j] the accumulator of lane j of that wave, for
       off = 32, 16, 8, 4, 2, 1 in that order: x[j] = x[j] + x[j+off] for
       every j < off. The wave's result y[w] is x[0].
    4. The result is (y[0] + y[2]) + (y[1] + y[3]).

    q: float32 [..., H]. Returns float32 [...].
    """
    q = np.asarray(q)
    if q.dtype != np.float32:
        raise TypeError("canonical_tree_sum expects float32")
    lead = q.shape[:-1]
    H = q.shape[-1]

    # steps 1-2: per-lane sequential chains
    acc = np.zeros(lead + (LANES,), dtype=np.float32)
    ngroups = -(-H // GROUP)
    for k in range(ngroups):
        lane = k % LANES
        for j in range(GROUP):
            h = GROUP * k + j
            if h >= H:
                break
            with np.errstate(over="ignore", invalid="ignore"):
                acc[..., lane] = np.add(acc[..., lane], q[..., h])

    # step 3: the halving tree inside each wave
    y = []
    for w in range(WAVES):
        x = acc[..., WAVE * w: WAVE * (w + 1)].copy()
        off = WAVE // 2
        while off >= 1:
            with np.errstate(over="ignore", invalid="ignore"):
                x[..., :off] = np.add(x[..., :off], x[..., off:2 * off])
            off //= 2
        y.append(x[..., 0].copy())

    # step 4: across the four waves
    with np.errstate(over="ignore", invalid="ignore"):
        return np.add(np.add(y[0], y[2]), np.add(y[1], y[3]))


def grad_pre_ref(residual: np.ndarray, grad_out: np.ndarray) -> np.ndarray:
    """grad_pre[t,i] = canonical_tree_sum over h of grad_out[t,h]*residual[t,i,h].

    Returns float32 [T,4].
    """
    return canonical_tree_sum(grad_pre_products(residual, grad_out))


def h_aggregate_bwd(residual: np.ndarray, pre: np.ndarray, grad_out: np.ndarray
                    ) -> tuple[np.ndarray, np.ndarray]:
    """Backward of h_aggregate_fwd. Returns (grad_residual uint16 [T,4,H],
    grad_pre float32 [T,4])."""
    _check_bwd_args(residual, pre, grad_out)
    return grad_residual_ref(pre, grad_out), grad_pre_ref(residual, grad_out)


def h_aggregate_bwd_acc(residual: np.ndarray, pre: np.ndarray, grad_out: np.ndarray,
                        grad_residual_in: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Backward that accumulates into an existing grad_residual (see
    grad_residual_acc_ref) and writes grad_pre. Returns (updated
    grad_residual uint16 [T,4,H], grad_pre float32 [T,4])."""
    _check_bwd_args(residual, pre, grad_out)
    if grad_residual_in.dtype != np.uint16 or grad_residual_in.shape != residual.shape:
        raise ValueError("grad_residual_in must be uint16 bf16 bits of shape [T, 4, H]")
    return (grad_residual_acc_ref(pre, grad_out, grad_residual_in),
            grad_pre_ref(residual, grad_out))


def grad_pre_exact(residual: np.ndarray, grad_out: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """fp64 sum over h of grad_out*residual_i, and of its absolute values.

    Used only to check the oracle: the terms are exact fp32 products, their
    fp64 sum has a relative error below H * 2**-53 of sum |q|.
    """
    _check_bwd_args(residual, np.zeros(residual.shape[:2], np.float32), grad_out)
    q = grad_pre_products(residual, grad_out).astype(np.float64)
    return q.sum(axis=-1), np.abs(q).sum(axis=-1)


# ---------------------------------------------------------------------------
# bf16 ulp and the fp64 acceptance rule for the forward
# ---------------------------------------------------------------------------

def bf16_ulp(bits: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at the magnitude of the given bf16 values.

    ulp(v) = 2**(max(floor(log2|v|), -126) - 7); ulp(0) = 2**-133 (the bf16
    subnormal spacing). Returned as float64.
    """
    v = widen_bf16(np.asarray(bits, dtype=np.uint16)).astype(np.float64)
    _, e = np.frexp(np.abs(v))                 # |v| = m * 2**e, m in [0.5, 1)
    expo = np.where(v == 0.0, -126, np.maximum(e - 1, -126))
    return np.ldexp(1.0, expo - 7)


def fwd_error_bound(out_bits: np.ndarray, mag: np.ndarray, n: int = HC) -> np.ndarray:
    """Largest |out - exact| the forward may show, per element.

    The fp32 evaluation has depth d = 1 + log2(n) (one product, then log2(n)
    levels of sums: 3 for the page's n = 4), so its error is at most
    ((1+u)**d - 1) * sum|pre_i r_i| with u = 2**-24, plus d * 2**-150 for
    results in the subnormal range; one bf16 rounding adds at most half a
    bf16 ulp of the result. A further (n+1) * 2**-53 * sum|pre_i r_i| covers
    the fp64 reference's own rounding.
    """
    u = 2.0 ** -24
    depth = 1 + int(np.log2(n))
    gamma = (1.0 + u) ** depth - 1.0
    return 0.5 * bf16_ulp(out_bits) + (gamma + (n + 1) * 2.0 ** -53) * mag + depth * 2.0 ** -150


def classify_fwd(out_bits: np.ndarray, exact: np.ndarray, mag: np.ndarray, n: int = HC) -> dict:
    """Count forward outputs within 1 bf16 ulp of the fp64 value, beyond 1 ulp
    but inside fwd_error_bound (cancellation), and outside both (a failure)."""
    out = widen_bf16(out_bits).astype(np.float64)
    err = np.abs(out - exact)
    ulp = bf16_ulp(out_bits)
    within_ulp = err <= ulp
    within_bound = err <= fwd_error_bound(out_bits, mag, n)
    return {
        "within_1ulp": int(within_ulp.sum()),
        "cancellation_bound": int((~within_ulp & within_bound).sum()),
        "fail": int((~within_ulp & ~within_bound).sum()),
    }


def tree_error_bound(H: int) -> float:
    """Relative error bound (to sum|q|) of canonical_tree_sum for length H.

    A term passes through at most ceil(H / (8*256)) * 8 chain additions, 6
    wave levels and 2 block levels; each rounding costs at most u = 2**-24.
    """
    depth = -(-H // (GROUP * LANES)) * GROUP + 6 + 2
    u = 2.0 ** -24
    return (1.0 + u) ** depth - 1.0


__all__ = [
    "HC", "SUPPORTED_HC", "GROUP", "LANES", "WAVE", "WAVES",
    "widen_bf16", "bf16_rne", "pairwise_tree",
    "h_aggregate_fwd", "h_aggregate_fwd_n", "h_aggregate_fwd_exact",
    "grad_residual_ref", "grad_residual_acc_ref", "grad_pre_products", "canonical_tree_sum",
    "grad_pre_ref", "h_aggregate_bwd", "h_aggregate_bwd_acc", "grad_pre_exact",
    "bf16_ulp", "fwd_error_bound", "classify_fwd", "tree_error_bound",
]

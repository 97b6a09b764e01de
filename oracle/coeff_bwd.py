"""Plain CPU oracle of the mHC coefficient backward epilogue.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline use it. It shares no code, header, helper, table or constant
generator with the HIP path.

Source: "perf: fuse mHC coefficient backward epilogue" (Liger-Kernel pull
request 1402).

* Section *Summary*: between the Sinkhorn backward and the fused MM/RMS
  backward sits an epilogue over the coefficient columns (24 of them at
  HC = 4). It forms the derivatives of the pre and post sigmoids, grad_mix,
  and fp32 partial sums for grad_b and the alpha gradients; a deterministic
  reducer turns the partials into the 24 grad_b columns and the three scalar
  alpha gradients.
* Section *Risks and Limitations*: both reductions run in a fixed
  two-stage order.
* Section *Performance Method*: batch B = 4, HC = 4, T in {128, 512, 2048}
  tokens; HC in {2, 8} as controls.

The page prints none of the formulas. The reading taken here (the plainest
one its parts support; PARITY UNPINNED against the page, since the page
gives nothing to compare with; the oracle is pinned to the calculus of this
reading instead):

* Columns. With expansion n the coefficient row has m = 2n + n*n columns
  (24 at n = 4): columns [0, n) are pre, [n, 2n) post, [2n, m) the n x n
  residual-mixing logits in row-major order. Group k(j) is 0, 1, 2 for the
  three kinds.
* Forward being differentiated: z[r, j] = alpha[k(j)] * mix[r, j] + b[j]
  (one scalar gain per group, one bias per column: "24 grad_b columns and
  three scalar alpha gradients"); pre = sigmoid(z_pre); post =
  c * sigmoid(z_post) with the scale c a parameter (the page does not fix
  it); z_res goes on to the Sinkhorn normalisation, whose backward delivers
  grad_res = dL/dz_res.
* The epilogue gets mix, the saved activations pre and post, the upstream
  gradients grad_pre, grad_post, grad_res, alpha[3] and c, and computes
    d[r, j] = dL/dz[r, j]:
      pre  columns: grad_pre  * (pre  * (1 - pre))        sigmoid' = s(1-s)
      post columns: grad_post * (post * (1 - post / c))   (c s)' = c s(1-s), s = post / c
      res  columns: grad_res
    grad_mix[r, j] = alpha[k(j)] * d[r, j]
    grad_b[j]      = row_sum over r of d[r, j]
    grad_alpha[k]  = row_sum over r of e[r, k], where e[r, k] adds
                     d[r, j] * mix[r, j] over the columns j of group k in
                     ascending j, starting from +0.0.
  The post gate's sigmoid is recovered from its saved output as post / c,
  one fp32 division rounded to nearest even (the plain derivative of
  post = c * sigmoid(z), written in the saved output). Every product,
  quotient, sum and difference is one fp32 round-to-nearest operation,
  evaluated in exactly the nesting written above.
* row_sum is this repository's fixed two-stage order (see `row_sum`); it
  depends only on the number of rows.

* Input precision (page section Testing Done: the sibling implementation's
  tests run FP16, BF16 and FP32 inputs; section Performance Method: BF16 is
  the primary matrix). With 16-bit inputs (`coeff_bwd_typed`), the six row
  tensors mix, pre, post, grad_pre, grad_post and grad_res are bf16 or fp16
  bit patterns; each value is widened to fp32 exactly, the computation above
  runs unchanged in fp32, grad_mix is rounded once to the input's format
  (round to nearest even, subnormals kept, overflow to infinity), and alpha,
  grad_b and grad_alpha stay fp32 (the page's fp32 partial sums).

Arithmetic model: as in oracle.h_aggregate, every fp32 operation is one
numpy float32 ufunc call; numpy vectorises only across independent rows or
columns. No np.sum, np.dot or einsum appears in an fp32 path.
"""

from __future__ import annotations

import math

import numpy as np

from oracle.h_aggregate import bf16_rne, widen_bf16

# Rows per first-stage chunk and lanes of the second stage of row_sum.
CHUNK = 64
LANES = 64

SUPPORTED_HC = (2, 4, 8)


def columns(n: int) -> int:
    """Coefficient columns at expansion n: n pre, n post, n*n residual."""
    return 2 * n + n * n


def groups(n: int) -> np.ndarray:
    """Group k(j) of every column j: 0 pre, 1 post, 2 residual mixing."""
    return np.array([0] * n + [1] * n + [2] * (n * n), dtype=np.int64)


def _halving_tree(x: np.ndarray) -> np.ndarray:
    """Fixed fp32 tree over axis -1 of length 64: for off = 32, 16, 8, 4, 2,
    1 in turn, x[i] = x[i] + x[i + off] for every i < off; returns x[0]."""
    x = x.copy()
    assert x.shape[-1] == 64
    off = 32
    while off >= 1:
        with np.errstate(over="ignore", invalid="ignore"):
            x[..., :off] = np.add(x[..., :off], x[..., off:2 * off])
        off //= 2
    return x[..., 0].copy()


def row_sum(x: np.ndarray) -> np.ndarray:
    """Fixed-order fp32 sum over axis 0 (the rows) of x [R, V] -> [V].

    Stage 1: the rows are cut into chunks of 64 consecutive rows (chunk c
    holds rows 64c .. 64c+63; rows past R count as +0.0) and each chunk is
    summed by the halving tree (offsets 32, 16, 8, 4, 2, 1) into P[c].
    Stage 2: 64 accumulators start at +0.0; the chunk sums are visited in
    ascending c, P[c] being added to accumulator c mod 64; the 64
    accumulators are then summed by the same halving tree.
    """
    x = np.asarray(x)
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError("row_sum expects float32 [R, V]")
    R, V = x.shape
    C = -(-R // CHUNK)
    padded = np.zeros((C * CHUNK, V), dtype=np.float32)
    padded[:R] = x
    # stage 1: [C, V, 64] so the tree runs over the chunk's rows
    P = _halving_tree(padded.reshape(C, CHUNK, V).transpose(0, 2, 1))   # [C, V]
    # stage 2
    acc = np.zeros((V, LANES), dtype=np.float32)
    for c in range(C):
        with np.errstate(over="ignore", invalid="ignore"):
            acc[:, c % LANES] = np.add(acc[:, c % LANES], P[c])
    return _halving_tree(acc)


def _check(mix, pre, post, grad_pre, grad_post, grad_res, alpha, n):
    if n not in SUPPORTED_HC:
        raise ValueError(f"n must be one of {SUPPORTED_HC}")
    m = columns(n)
    R = mix.shape[0]
    want = {"mix": (mix, (R, m)), "pre": (pre, (R, n)), "post": (post, (R, n)),
            "grad_pre": (grad_pre, (R, n)), "grad_post": (grad_post, (R, n)),
            "grad_res": (grad_res, (R, n * n)), "alpha": (alpha, (3,))}
    for name, (a, shape) in want.items():
        if a.dtype != np.float32 or a.shape != shape:
            raise ValueError(f"{name} must be float32 of shape {shape}, got {a.dtype} {a.shape}")
    return R, m


def dz(pre, post, grad_pre, grad_post, grad_res, post_scale) -> np.ndarray:
    """d[r, j] = dL/dz[r, j] for all m columns, float32 [R, m]."""
    one = np.float32(1.0)
    with np.errstate(over="ignore", invalid="ignore", under="ignore", divide="ignore"):
        d_pre = np.multiply(grad_pre, np.multiply(pre, np.subtract(one, pre)))
        s = np.divide(post, np.float32(post_scale))      # the post gate's sigmoid
        d_post = np.multiply(grad_post, np.multiply(post, np.subtract(one, s)))
    return np.concatenate([d_pre, d_post, grad_res], axis=1).astype(np.float32)


def coeff_bwd(mix, pre, post, grad_pre, grad_post, grad_res, alpha, post_scale, n
              ) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """The epilogue as defined in the module docstring.

    Returns (grad_mix float32 [R, m], grad_b float32 [m], grad_alpha float32 [3]).
    """
    R, m = _check(mix, pre, post, grad_pre, grad_post, grad_res, alpha, n)
    d = dz(pre, post, grad_pre, grad_post, grad_res, post_scale)
    k = groups(n)
    with np.errstate(over="ignore", invalid="ignore", under="ignore"):
        grad_mix = np.multiply(alpha[k][None, :], d)
        prod = np.multiply(d, mix)                         # [R, m]
        e = np.zeros((R, 3), dtype=np.float32)
        for j in range(m):                                 # ascending j within each group
            e[:, k[j]] = np.add(e[:, k[j]], prod[:, j])
    grad_b = row_sum(d)
    grad_alpha = row_sum(e)
    return grad_mix.astype(np.float32), grad_b, grad_alpha


# Storage formats of the six row tensors and grad_mix.
DTYPES = ("f32", "bf16", "f16")
ROW_INPUTS = ("mix", "pre", "post", "grad_pre", "grad_post", "grad_res")


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float32, exactly: f32 as is; bf16 and f16 from their
    uint16 bit patterns (every bf16 and fp16 value is an fp32 value)."""
    if dtype == "f32":
        if x.dtype != np.float32:
            raise ValueError("f32 tensors must be float32")
        return x
    if x.dtype != np.uint16:
        raise ValueError(f"{dtype} tensors must be uint16 bit patterns")
    if dtype == "bf16":
        return widen_bf16(x)
    if dtype == "f16":
        with np.errstate(invalid="ignore"):
            return x.view(np.float16).astype(np.float32)
    raise ValueError(f"dtype must be one of {DTYPES}")


def narrow(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> the stored format, rounded to nearest even (subnormals
    kept, overflow to infinity): f32 unchanged; bf16 and f16 as uint16 bit
    patterns."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return bf16_rne(x)
    if dtype == "f16":
        with np.errstate(over="ignore"):
            return x.astype(np.float16).view(np.uint16)
    raise ValueError(f"dtype must be one of {DTYPES}")


def coeff_bwd_typed(mix, pre, post, grad_pre, grad_post, grad_res, alpha, post_scale, n,
                    dtype: str) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """The epilogue on stored inputs of the given format: the six row
    tensors widened exactly, coeff_bwd in fp32, grad_mix narrowed once.

    Returns (grad_mix [R, m] in the stored format, grad_b float32 [m],
    grad_alpha float32 [3])."""
    rows = [widen(np.asarray(t), dtype) for t in (mix, pre, post, grad_pre, grad_post, grad_res)]
    gm, gb, ga = coeff_bwd(*rows, alpha, post_scale, n)
    return narrow(gm, dtype), gb, ga


def coeff_bwd_exact(mix, pre, post, grad_pre, grad_post, grad_res, alpha, post_scale, n
                    ) -> dict[str, np.ndarray]:
    """fp64 values of the same quantities (from the same fp32 inputs), with
    correctly rounded sums (math.fsum), and per-element magnitudes that bound
    the fp32 evaluation error without cancellation:

      d, grad_mix [R, m]; grad_b [m]; grad_alpha [3];
      mag_d [R, m]   with |fp32 d - d| <= 5 u mag_d   (u = 2^-24)
      mag_b [m], mag_alpha [3]: sums of the magnitudes of the summed terms.
    """
    R, m = _check(mix, pre, post, grad_pre, grad_post, grad_res, alpha, n)
    f = lambda a: np.asarray(a, dtype=np.float64)
    p, q, gp, gq, gr, mx, al = map(f, (pre, post, grad_pre, grad_post, grad_res, mix, alpha))
    c = float(np.float32(post_scale))
    s = q / c
    d = np.concatenate([gp * (p * (1.0 - p)), gq * (q * (1.0 - s)), gr], axis=1)
    mag_d = np.concatenate([np.abs(gp) * np.abs(p) * (1.0 + np.abs(p)),
                            np.abs(gq) * np.abs(q) * (1.0 + np.abs(s)),
                            np.abs(gr)], axis=1)
    k = groups(n)
    grad_mix = al[k][None, :] * d
    grad_b = np.array([math.fsum(d[:, j]) for j in range(m)])
    mag_b = np.array([math.fsum(mag_d[:, j]) for j in range(m)])
    grad_alpha = np.zeros(3)
    mag_alpha = np.zeros(3)
    for g in range(3):
        cols = np.nonzero(k == g)[0]
        grad_alpha[g] = math.fsum((d[:, cols] * mx[:, cols]).ravel())
        mag_alpha[g] = math.fsum((mag_d[:, cols] * np.abs(mx[:, cols])).ravel())
    return dict(d=d, grad_mix=grad_mix, grad_b=grad_b, grad_alpha=grad_alpha,
                mag_d=mag_d, mag_b=mag_b, mag_alpha=mag_alpha)


def row_sum_depth(R: int) -> int:
    """Longest chain of fp32 additions any one term passes through in
    row_sum over R rows: 6 tree levels, one add per chunk sum visited by its
    accumulator, 6 tree levels."""
    C = -(-R // CHUNK)
    return 6 + max(1, -(-C // LANES)) + 6


def reduction_error_bound(R: int, group_width: int = 1) -> float:
    """Relative (to the sum of magnitudes) bound of row_sum on top of the
    per-term errors: gamma_k = k u / (1 - k u) for the chain length k, plus
    the sequential sum over the group's columns for the alpha terms."""
    u = 2.0 ** -24
    k = row_sum_depth(R) + group_width
    return k * u / (1.0 - k * u)

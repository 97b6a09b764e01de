"""Seeded synthetic inputs for the h_aggregate forward and backward.

Shared by the tests, the benchmark and the smoke check. It holds none of the
operation's arithmetic: it only draws random numbers and stores them in the
operation's input formats (bf16 bit patterns via torch's CPU conversion,
fp32 as drawn).

Recipe (the pages print no value distributions; these follow the shapes of
the page "Add batch-invariant h_aggregate kernel", sections Correctness and
Performance):
  rng = numpy.random.default_rng(seed)      (PCG64), draws in this order:
  residual [T,n,H] = bf16(rng.standard_normal(float32))   n = 4 (or 2, 8)
  pre      [T,n]   = rng.random(float32)                 U[0,1), gate-like
  grad_out [T,H]   = bf16(rng.normal(0, 0.1) as float32)   (if requested)
  outliers         = rng.random((T,4,H)) < 0.01 scales residual by 64 before
                     the bf16 conversion (if requested; exact power of two)
"""

from __future__ import annotations

import numpy as np
import torch

HC = 4


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns, through torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def make_inputs(T: int, H: int, seed: int = 0, *, grad: bool = False,
                outliers: bool = False, hc: int = HC) -> dict[str, np.ndarray]:
    """Host inputs: residual (uint16 [T,hc,H]), pre (float32 [T,hc]) and,
    if grad, grad_out (uint16 [T,H]). hc is the expansion rate (4 on the
    page; 2 and 8 for the generalised operation)."""
    rng = np.random.default_rng(seed)
    res = rng.standard_normal((T, hc, H), dtype=np.float32)
    pre = rng.random((T, hc), dtype=np.float32)
    out = {"pre": pre}
    if grad:
        out["grad_out"] = to_bf16_bits(rng.normal(0.0, 0.1, (T, H)).astype(np.float32))
    if outliers:
        mask = rng.random((T, hc, H)) < 0.01
        res = np.where(mask, res * np.float32(64.0), res).astype(np.float32)
    out["residual"] = to_bf16_bits(res)
    return out


def make_unit_inputs_device(T: int, H: int, seed: int, device, hc: int = HC
                            ) -> dict[str, torch.Tensor]:
    """Device inputs whose backward reduction is exact in any order, drawn on
    the device (for sizes the host would take minutes to draw) with a
    torch.Generator seeded with `seed`, in this order: residual codes
    (uint8 in [0, 16): 0 -> -1, 1 -> +1, otherwise 0, so 1/8 of the entries
    are non-zero), grad_out signs (+1 or -1), pre U[0,1) fp32. Values are
    written as bf16 bit patterns directly (+1 is 0x3F80, -1 is 0xBF80)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    code = torch.randint(0, 16, (T, hc, H), dtype=torch.uint8, device=device, generator=gen)
    plus = torch.tensor(0x3F80, dtype=torch.int16, device=device)
    minus = torch.tensor(0xBF80 - 0x10000, dtype=torch.int16, device=device)
    zero = torch.tensor(0, dtype=torch.int16, device=device)
    residual = torch.where(code == 1, plus, torch.where(code == 0, minus, zero))
    del code
    signs = torch.randint(0, 2, (T, H), dtype=torch.uint8, device=device, generator=gen)
    grad_out = torch.where(signs == 1, plus, minus)
    pre = torch.rand((T, hc), dtype=torch.float32, device=device, generator=gen)
    return {"residual": residual.view(torch.bfloat16), "pre": pre,
            "grad_out": grad_out.view(torch.bfloat16)}


def make_coeff_unit_inputs_device(rows: int, n: int, seed: int, device
                                  ) -> dict[str, torch.Tensor]:
    """Device inputs of the coefficient epilogue whose sums are exact in any
    order, drawn on the device with a torch.Generator seeded with `seed`, in
    this order: mix sign codes (uint8 0/1 -> -1/+1, every column), residual
    gradient codes (uint8 in [0, 128): 0 -> -1, 1 -> +1, otherwise 0), pre
    U[0,1), post U[0,2). grad_pre and grad_post are zero. The uint8 codes
    are returned too ("mix_code", "grad_res_code") so that a checker can form
    exact integer sums without reading the fp32 tensors back."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    m = 2 * n + n * n
    one = torch.tensor(1.0, dtype=torch.float32, device=device)
    zero = torch.tensor(0.0, dtype=torch.float32, device=device)
    mix_code = torch.randint(0, 2, (rows, m), dtype=torch.uint8, device=device, generator=gen)
    mix = torch.where(mix_code == 1, one, -one)
    res_code = torch.randint(0, 128, (rows, n * n), dtype=torch.uint8, device=device,
                             generator=gen)
    grad_res = torch.where(res_code == 1, one, torch.where(res_code == 0, -one, zero))
    pre = torch.rand((rows, n), dtype=torch.float32, device=device, generator=gen)
    post = torch.rand((rows, n), dtype=torch.float32, device=device, generator=gen) * 2.0
    return {"mix": mix, "pre": pre, "post": post,
            "grad_pre": torch.zeros((rows, n), dtype=torch.float32, device=device),
            "grad_post": torch.zeros((rows, n), dtype=torch.float32, device=device),
            "grad_res": grad_res,
            "alpha": torch.tensor([0.75, 1.25, 1.5], dtype=torch.float32, device=device),
            "mix_code": mix_code, "grad_res_code": res_code}


def make_coeff_inputs(rows: int, n: int = HC, seed: int = 0, *,
                      post_scale: float = 2.0) -> dict[str, np.ndarray]:
    """Host inputs of the coefficient backward epilogue (all float32).

    Recipe (the page "perf: fuse mHC coefficient backward epilogue" gives the
    shapes, B = 4 sequences of T in {128, 512, 2048} tokens at HC = 4, but no
    value distributions): rng = numpy.random.default_rng(seed), drawing in
    this order: mix [R, m] standard normal (m = 2n + n*n); pre [R, n] U[0,1)
    (a sigmoid output); post [R, n] U[0,1) times post_scale (a scaled
    sigmoid output); grad_pre, grad_post [R, n] and grad_res [R, n*n]
    standard normal; alpha [3] U[0.5, 1.5).
    """
    rng = np.random.default_rng(seed)
    m = 2 * n + n * n
    f = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    return {
        "mix": f(rng.standard_normal((rows, m), dtype=np.float32)),
        "pre": f(rng.random((rows, n), dtype=np.float32)),
        "post": f(rng.random((rows, n), dtype=np.float32) * np.float32(post_scale)),
        "grad_pre": f(rng.standard_normal((rows, n), dtype=np.float32)),
        "grad_post": f(rng.standard_normal((rows, n), dtype=np.float32)),
        "grad_res": f(rng.standard_normal((rows, n * n), dtype=np.float32)),
        "alpha": f(rng.uniform(0.5, 1.5, 3)),
    }


def bits_to_bf16_tensor(bits: np.ndarray, device="cpu") -> torch.Tensor:
    """uint16 bf16 patterns -> torch.bfloat16 tensor (same bits)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def bf16_tensor_to_bits(t: torch.Tensor) -> np.ndarray:
    """torch.bfloat16 (any device) -> uint16 bit patterns on the host."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16).copy()


def to_device(inputs: dict[str, np.ndarray], device) -> dict[str, torch.Tensor]:
    """Copy host inputs to the device with identical bytes."""
    out = {}
    for k, v in inputs.items():
        if v.dtype == np.uint16:
            out[k] = bits_to_bf16_tensor(v, device)
        else:
            out[k] = torch.from_numpy(np.ascontiguousarray(v)).to(device)
    return out

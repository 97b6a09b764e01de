"""Python binding of the coefficient backward epilogue: argument marshalling
only.

Checks the tensors' device, dtype, shape and layout, allocates outputs and
the workspace through torch when the caller gives none, and hands raw device
pointers, sizes and torch's current HIP stream to the C ABI
(include/mhc_coeff_bwd.h, which states the operation). All arithmetic runs
in the gfx950 kernels; a missing library raises ImportError.

Operation: the epilogue of the page "perf: fuse mHC coefficient backward
epilogue" (Liger-Kernel pull request 1402), section Summary, in the reading
the header states.
"""

from __future__ import annotations

import torch

from . import _lib
from ._lib import check_coeff
from .ops import _require, _stream_handle

SUPPORTED_HC = (2, 4, 8)


def coeff_columns(n: int) -> int:
    """Coefficient columns at expansion n: n pre, n post, n*n residual."""
    return 2 * n + n * n


def mhc_coeff_bwd_workspace_bytes(rows: int, n: int) -> int:
    """Workspace bytes a call with `rows` rows at expansion n needs."""
    got = _lib.coeff_lib().mhc_coeff_bwd_workspace_bytes(int(rows), int(n))
    if got < 0:
        raise ValueError(f"invalid rows={rows} or n={n}")
    return int(got)


def mhc_coeff_bwd_plan(rows: int, n: int, launches: int = 0) -> int:
    """Launches (1 or 2) a call with these arguments makes."""
    got = _lib.coeff_lib().mhc_coeff_bwd_plan(int(rows), int(n), int(launches))
    if got < 0:
        raise ValueError(f"invalid rows={rows}, n={n} or launches={launches}")
    return int(got)


def mhc_coeff_bwd_validate(mix: int, pre: int, post: int, grad_pre: int, grad_post: int,
                           grad_res: int, alpha: int, post_scale: float, grad_mix: int,
                           grad_b: int, grad_alpha: int, workspace: int, workspace_bytes: int,
                           rows: int, n: int) -> None:
    """Host-only argument check on raw addresses (no device access)."""
    check_coeff(_lib.coeff_lib().mhc_coeff_bwd_validate(
        mix, pre, post, grad_pre, grad_post, grad_res, alpha, float(post_scale), grad_mix,
        grad_b, grad_alpha, workspace, int(workspace_bytes), int(rows), int(n)))


_FORMATS = {torch.float32: _lib.MHC_COEFF_F32, torch.bfloat16: _lib.MHC_COEFF_BF16,
            torch.float16: _lib.MHC_COEFF_F16}


def mhc_coeff_bwd(mix: torch.Tensor, pre: torch.Tensor, post: torch.Tensor,
                  grad_pre: torch.Tensor, grad_post: torch.Tensor, grad_res: torch.Tensor,
                  alpha: torch.Tensor, post_scale: float, *, grad_mix: torch.Tensor | None = None,
                  grad_b: torch.Tensor | None = None, grad_alpha: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, launches: int = 0,
                  stream: torch.cuda.Stream | None = None, start_event=None, stop_event=None
                  ) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """(grad_mix [R, m], grad_b [m], grad_alpha [3]) from mix [R, m], pre,
    post, grad_pre, grad_post [R, n], grad_res [R, n*n] (all fp32, all
    bf16 or all fp16: the storage format, which grad_mix takes too), alpha
    [3] fp32 and the post-gate scale; grad_b and grad_alpha are fp32.
    Asynchronous on `stream`. A workspace given by the caller must have been
    zeroed once (its first 4 bytes are the arrival counter every completed
    call leaves at zero); without one, a zeroed workspace is allocated.
    launches: 0 (policy), 1 or 2. start_event / stop_event are raw
    hipEvent_t handles (or None)."""
    if not isinstance(pre, torch.Tensor) or pre.dim() != 2 or pre.shape[1] not in SUPPORTED_HC:
        raise ValueError("pre must have shape [R, n] with n in (2, 4, 8)")
    if pre.dtype not in _FORMATS:
        raise TypeError(f"the row tensors must be float32, bfloat16 or float16 (got {pre.dtype})")
    R, n = int(pre.shape[0]), int(pre.shape[1])
    m = coeff_columns(n)
    dev = pre.device
    dt = pre.dtype
    f32 = torch.float32
    _require(pre, "pre", dt, (R, n))
    _require(mix, "mix", dt, (R, m), dev)
    _require(post, "post", dt, (R, n), dev)
    _require(grad_pre, "grad_pre", dt, (R, n), dev)
    _require(grad_post, "grad_post", dt, (R, n), dev)
    _require(grad_res, "grad_res", dt, (R, n * n), dev)
    _require(alpha, "alpha", f32, (3,), dev)
    if grad_mix is None:
        grad_mix = torch.empty((R, m), dtype=dt, device=dev)
    if grad_b is None:
        grad_b = torch.empty((m,), dtype=f32, device=dev)
    if grad_alpha is None:
        grad_alpha = torch.empty((3,), dtype=f32, device=dev)
    _require(grad_mix, "grad_mix", dt, (R, m), dev)
    _require(grad_b, "grad_b", f32, (m,), dev)
    _require(grad_alpha, "grad_alpha", f32, (3,), dev)
    need = mhc_coeff_bwd_workspace_bytes(R, n)
    if workspace is None:
        workspace = torch.zeros((max(need, 1),), dtype=torch.uint8, device=dev)
    if not isinstance(workspace, torch.Tensor) or workspace.device != dev or \
            not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    ws_bytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        st = _lib.coeff_lib().mhc_coeff_bwd_ex(
            mix.data_ptr(), pre.data_ptr(), post.data_ptr(), grad_pre.data_ptr(),
            grad_post.data_ptr(), grad_res.data_ptr(), alpha.data_ptr(), float(post_scale),
            grad_mix.data_ptr(), grad_b.data_ptr(), grad_alpha.data_ptr(), workspace.data_ptr(),
            ws_bytes, R, n, _FORMATS[dt], int(launches), _stream_handle(dev, stream),
            start_event, stop_event)
    check_coeff(st)
    return grad_mix, grad_b, grad_alpha

"""Python binding of the h_aggregate library: argument marshalling only.

Every function here checks the tensors' device, dtype, shape and layout,
then hands raw device pointers, sizes and torch's current HIP stream to the
C ABI (include/mhc_h_aggregate.h). All arithmetic happens in the gfx950
kernels; PyTorch provides device memory and streams. There is no fallback:
a missing library raises ImportError, a non-GPU tensor raises TypeError.

Operation: page "Add batch-invariant h_aggregate kernel" (RL-Kernel pull
request 366), sections Summary and Batch invariance; backward requested in
that page's review comments.
"""

from __future__ import annotations

import ctypes
from typing import Mapping

import torch

from . import _lib
from ._lib import check, mhc_launch

HC = 4


def _stream_handle(device: torch.device, stream: torch.cuda.Stream | None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return int(s.cuda_stream)


def _launch_arg(launch) -> ctypes.c_void_p | ctypes._Pointer | None:
    if launch is None:
        return None
    if isinstance(launch, mhc_launch):
        return ctypes.pointer(launch)
    if isinstance(launch, Mapping):
        return ctypes.pointer(mhc_launch(**{k: int(v) for k, v in launch.items()}))
    raise TypeError("launch must be None, an mhc_launch or a mapping of its fields")


def _require(t: torch.Tensor, name: str, dtype: torch.dtype, shape: tuple, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise TypeError(f"{name} must be on a GPU (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _fwd_shapes(residual: torch.Tensor) -> tuple[int, int]:
    if not isinstance(residual, torch.Tensor) or residual.dim() != 3 or residual.shape[1] != HC:
        raise ValueError("residual must have shape [T, 4, H]")
    return int(residual.shape[0]), int(residual.shape[2])


# ---------------------------------------------------------------------------
# Names of the C ABI
# ---------------------------------------------------------------------------

def mhc_h_aggregate_fwd(residual: torch.Tensor, pre: torch.Tensor, out: torch.Tensor,
                        stream: torch.cuda.Stream | None = None, launch=None) -> torch.Tensor:
    """out[T,H] bf16 <- h_aggregate(residual[T,4,H] bf16, pre[T,4] fp32). Asynchronous."""
    T, H = _fwd_shapes(residual)
    dev = residual.device
    _require(residual, "residual", torch.bfloat16, (T, HC, H))
    _require(pre, "pre", torch.float32, (T, HC), dev)
    _require(out, "out", torch.bfloat16, (T, H), dev)
    with torch.cuda.device(dev):
        st = _lib.lib().mhc_h_aggregate_fwd_ex(
            residual.data_ptr(), pre.data_ptr(), out.data_ptr(), T, H,
            _stream_handle(dev, stream), _launch_arg(launch))
    check(st)
    return out


def mhc_h_aggregate_bwd(residual: torch.Tensor, pre: torch.Tensor, grad_out: torch.Tensor,
                        grad_residual: torch.Tensor, grad_pre: torch.Tensor,
                        stream: torch.cuda.Stream | None = None, launch=None
                        ) -> tuple[torch.Tensor, torch.Tensor]:
    """(grad_residual[T,4,H] bf16, grad_pre[T,4] fp32) <- backward. Asynchronous.

    Both outputs are overwritten, never accumulated into.
    """
    T, H = _fwd_shapes(residual)
    dev = residual.device
    _require(residual, "residual", torch.bfloat16, (T, HC, H))
    _require(pre, "pre", torch.float32, (T, HC), dev)
    _require(grad_out, "grad_out", torch.bfloat16, (T, H), dev)
    _require(grad_residual, "grad_residual", torch.bfloat16, (T, HC, H), dev)
    _require(grad_pre, "grad_pre", torch.float32, (T, HC), dev)
    with torch.cuda.device(dev):
        st = _lib.lib().mhc_h_aggregate_bwd_ex(
            residual.data_ptr(), pre.data_ptr(), grad_out.data_ptr(),
            grad_residual.data_ptr(), grad_pre.data_ptr(), T, H,
            _stream_handle(dev, stream), _launch_arg(launch))
    check(st)
    return grad_residual, grad_pre


def mhc_h_aggregate_fwd_timed(residual: torch.Tensor, pre: torch.Tensor, out: torch.Tensor,
                              start_event: int | None, stop_event: int | None,
                              stream: torch.cuda.Stream | None = None, launch=None
                              ) -> torch.Tensor:
    """Forward whose first / last kernel dispatch records the given raw
    hipEvent_t handles (ints; None for no event) at its own start / end."""
    T, H = _fwd_shapes(residual)
    dev = residual.device
    _require(residual, "residual", torch.bfloat16, (T, HC, H))
    _require(pre, "pre", torch.float32, (T, HC), dev)
    _require(out, "out", torch.bfloat16, (T, H), dev)
    with torch.cuda.device(dev):
        st = _lib.lib().mhc_h_aggregate_fwd_timed(
            residual.data_ptr(), pre.data_ptr(), out.data_ptr(), T, H,
            _stream_handle(dev, stream), _launch_arg(launch), start_event, stop_event)
    check(st)
    return out


def mhc_h_aggregate_bwd_timed(residual: torch.Tensor, pre: torch.Tensor, grad_out: torch.Tensor,
                              grad_residual: torch.Tensor, grad_pre: torch.Tensor,
                              start_event: int | None, stop_event: int | None,
                              stream: torch.cuda.Stream | None = None, launch=None
                              ) -> tuple[torch.Tensor, torch.Tensor]:
    """Backward whose first / last kernel dispatch records the given raw
    hipEvent_t handles at its own start / end."""
    T, H = _fwd_shapes(residual)
    dev = residual.device
    _require(residual, "residual", torch.bfloat16, (T, HC, H))
    _require(pre, "pre", torch.float32, (T, HC), dev)
    _require(grad_out, "grad_out", torch.bfloat16, (T, H), dev)
    _require(grad_residual, "grad_residual", torch.bfloat16, (T, HC, H), dev)
    _require(grad_pre, "grad_pre", torch.float32, (T, HC), dev)
    with torch.cuda.device(dev):
        st = _lib.lib().mhc_h_aggregate_bwd_timed(
            residual.data_ptr(), pre.data_ptr(), grad_out.data_ptr(),
            grad_residual.data_ptr(), grad_pre.data_ptr(), T, H,
            _stream_handle(dev, stream), _launch_arg(launch), start_event, stop_event)
    check(st)
    return grad_residual, grad_pre


def mhc_h_aggregate_bwd_acc(residual: torch.Tensor, pre: torch.Tensor, grad_out: torch.Tensor,
                            grad_residual: torch.Tensor, grad_pre: torch.Tensor,
                            stream: torch.cuda.Stream | None = None, launch=None,
                            start_event: int | None = None, stop_event: int | None = None
                            ) -> tuple[torch.Tensor, torch.Tensor]:
    """Accumulating backward: grad_residual += pre * grad_out (in place, one
    bf16 rounding of the fp32 sum); grad_pre is written. Asynchronous."""
    T, H = _fwd_shapes(residual)
    dev = residual.device
    _require(residual, "residual", torch.bfloat16, (T, HC, H))
    _require(pre, "pre", torch.float32, (T, HC), dev)
    _require(grad_out, "grad_out", torch.bfloat16, (T, H), dev)
    _require(grad_residual, "grad_residual", torch.bfloat16, (T, HC, H), dev)
    _require(grad_pre, "grad_pre", torch.float32, (T, HC), dev)
    with torch.cuda.device(dev):
        st = _lib.lib().mhc_h_aggregate_bwd_acc(
            residual.data_ptr(), pre.data_ptr(), grad_out.data_ptr(),
            grad_residual.data_ptr(), grad_pre.data_ptr(), T, H,
            _stream_handle(dev, stream), _launch_arg(launch), start_event, stop_event)
    check(st)
    return grad_residual, grad_pre


def _shapes_n(residual: torch.Tensor) -> tuple[int, int, int]:
    if not isinstance(residual, torch.Tensor) or residual.dim() != 3 or \
            residual.shape[1] not in (2, 4, 8):
        raise ValueError("residual must have shape [T, n, H] with n in {2, 4, 8}")
    return int(residual.shape[0]), int(residual.shape[1]), int(residual.shape[2])


def mhc_h_aggregate_fwd_n(residual: torch.Tensor, pre: torch.Tensor, out: torch.Tensor,
                          stream: torch.cuda.Stream | None = None, launch=None,
                          start_event: int | None = None, stop_event: int | None = None
                          ) -> torch.Tensor:
    """Forward for expansion rate n in {2, 4, 8}: residual [T,n,H], pre [T,n]."""
    T, n, H = _shapes_n(residual)
    dev = residual.device
    _require(residual, "residual", torch.bfloat16, (T, n, H))
    _require(pre, "pre", torch.float32, (T, n), dev)
    _require(out, "out", torch.bfloat16, (T, H), dev)
    with torch.cuda.device(dev):
        st = _lib.lib().mhc_h_aggregate_fwd_n(
            residual.data_ptr(), pre.data_ptr(), out.data_ptr(), T, n, H,
            _stream_handle(dev, stream), _launch_arg(launch), start_event, stop_event)
    check(st)
    return out


def mhc_h_aggregate_bwd_n(residual: torch.Tensor, pre: torch.Tensor, grad_out: torch.Tensor,
                          grad_residual: torch.Tensor, grad_pre: torch.Tensor,
                          accumulate: bool = False, stream: torch.cuda.Stream | None = None,
                          launch=None, start_event: int | None = None,
                          stop_event: int | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """Backward for expansion rate n in {2, 4, 8} (written or accumulating)."""
    T, n, H = _shapes_n(residual)
    dev = residual.device
    _require(residual, "residual", torch.bfloat16, (T, n, H))
    _require(pre, "pre", torch.float32, (T, n), dev)
    _require(grad_out, "grad_out", torch.bfloat16, (T, H), dev)
    _require(grad_residual, "grad_residual", torch.bfloat16, (T, n, H), dev)
    _require(grad_pre, "grad_pre", torch.float32, (T, n), dev)
    with torch.cuda.device(dev):
        st = _lib.lib().mhc_h_aggregate_bwd_n(
            residual.data_ptr(), pre.data_ptr(), grad_out.data_ptr(),
            grad_residual.data_ptr(), grad_pre.data_ptr(), T, n, H, 1 if accumulate else 0,
            _stream_handle(dev, stream), _launch_arg(launch), start_event, stop_event)
    check(st)
    return grad_residual, grad_pre


def _addr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    return int(x)


def mhc_h_aggregate_plan_fwd(residual, pre, out, T: int, H: int, launch=None) -> tuple[dict, int]:
    """Host-only: the launch shape and block count a forward call would use.

    Pointer arguments may be tensors or plain integers (only their numeric
    value is used, for alignment and overlap rules).
    """
    plan = mhc_launch()
    grid = ctypes.c_int64(0)
    check(_lib.lib().mhc_h_aggregate_plan_fwd(_addr(residual), _addr(pre), _addr(out), T, H,
                                              _launch_arg(launch), ctypes.byref(plan),
                                              ctypes.byref(grid)))
    return plan.as_dict(), int(grid.value)


def mhc_h_aggregate_plan_bwd(residual, pre, grad_out, grad_residual, grad_pre, T: int, H: int,
                             launch=None) -> tuple[dict, int]:
    """Host-only: the launch shape and block count a backward call would use."""
    plan = mhc_launch()
    grid = ctypes.c_int64(0)
    check(_lib.lib().mhc_h_aggregate_plan_bwd(_addr(residual), _addr(pre), _addr(grad_out),
                                              _addr(grad_residual), _addr(grad_pre), T, H,
                                              _launch_arg(launch), ctypes.byref(plan),
                                              ctypes.byref(grid)))
    return plan.as_dict(), int(grid.value)


def mhc_h_aggregate_plan_bwd_acc(residual, pre, grad_out, grad_residual, grad_pre, T: int,
                                 H: int, launch=None) -> tuple[dict, int]:
    """Host-only: the launch shape and block count an accumulating backward
    call would use."""
    plan = mhc_launch()
    grid = ctypes.c_int64(0)
    check(_lib.lib().mhc_h_aggregate_plan_bwd_acc(_addr(residual), _addr(pre), _addr(grad_out),
                                                  _addr(grad_residual), _addr(grad_pre), T, H,
                                                  _launch_arg(launch), ctypes.byref(plan),
                                                  ctypes.byref(grid)))
    return plan.as_dict(), int(grid.value)


def mhc_h_aggregate_plan_fwd_n(residual, pre, out, T: int, n: int, H: int,
                               launch=None) -> tuple[dict, int]:
    """Host-only: forward launch shape for expansion rate n."""
    plan = mhc_launch()
    grid = ctypes.c_int64(0)
    check(_lib.lib().mhc_h_aggregate_plan_fwd_n(_addr(residual), _addr(pre), _addr(out), T, n,
                                                H, _launch_arg(launch), ctypes.byref(plan),
                                                ctypes.byref(grid)))
    return plan.as_dict(), int(grid.value)


def mhc_h_aggregate_plan_bwd_n(residual, pre, grad_out, grad_residual, grad_pre, T: int,
                               n: int, H: int, accumulate: bool = False,
                               launch=None) -> tuple[dict, int]:
    """Host-only: backward launch shape for expansion rate n."""
    plan = mhc_launch()
    grid = ctypes.c_int64(0)
    check(_lib.lib().mhc_h_aggregate_plan_bwd_n(_addr(residual), _addr(pre), _addr(grad_out),
                                                _addr(grad_residual), _addr(grad_pre), T, n,
                                                H, 1 if accumulate else 0,
                                                _launch_arg(launch), ctypes.byref(plan),
                                                ctypes.byref(grid)))
    return plan.as_dict(), int(grid.value)


def mhc_h_aggregate_validate_fwd(residual, pre, out, T: int, H: int) -> int:
    """Host-only: status code a forward call would return before launching."""
    return int(_lib.lib().mhc_h_aggregate_validate_fwd(_addr(residual), _addr(pre), _addr(out),
                                                       T, H))


def mhc_h_aggregate_validate_bwd(residual, pre, grad_out, grad_residual, grad_pre,
                                 T: int, H: int) -> int:
    """Host-only: status code a backward call would return before launching."""
    return int(_lib.lib().mhc_h_aggregate_validate_bwd(
        _addr(residual), _addr(pre), _addr(grad_out), _addr(grad_residual), _addr(grad_pre),
        T, H))


# ---------------------------------------------------------------------------
# Allocating conveniences and autograd
# ---------------------------------------------------------------------------

def h_aggregate(residual: torch.Tensor, pre: torch.Tensor) -> torch.Tensor:
    """Forward with a freshly allocated output (no autograd); residual
    [T, n, H] with n in {2, 4, 8}."""
    T, n, H = _shapes_n(residual)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=residual.device)
    if n == HC:
        return mhc_h_aggregate_fwd(residual, pre, out)
    return mhc_h_aggregate_fwd_n(residual, pre, out)


def mhc_pre_h_aggregate(residual: torch.Tensor, pre: torch.Tensor) -> torch.Tensor:
    """The forward under the entry-point name the page's tests call (page
    "Add batch-invariant h_aggregate kernel", section Correctness): a
    freshly allocated out[T, H] bf16 from residual[T, n, H] bf16 and
    pre[T, n] fp32. Same as h_aggregate."""
    return h_aggregate(residual, pre)


def h_aggregate_backward(residual: torch.Tensor, pre: torch.Tensor, grad_out: torch.Tensor
                         ) -> tuple[torch.Tensor, torch.Tensor]:
    """Backward with freshly allocated gradients; residual [T, n, H] with n
    in {2, 4, 8}."""
    T, n, H = _shapes_n(residual)
    grad_residual = torch.empty((T, n, H), dtype=torch.bfloat16, device=residual.device)
    grad_pre = torch.empty((T, n), dtype=torch.float32, device=residual.device)
    if n == HC:
        return mhc_h_aggregate_bwd(residual, pre, grad_out, grad_residual, grad_pre)
    return mhc_h_aggregate_bwd_n(residual, pre, grad_out, grad_residual, grad_pre)


class HAggregate(torch.autograd.Function):
    """Autograd wrapper: forward and backward both run the gfx950 kernels
    (any supported expansion rate)."""

    @staticmethod
    def forward(ctx, residual: torch.Tensor, pre: torch.Tensor) -> torch.Tensor:
        ctx.save_for_backward(residual, pre)
        return h_aggregate(residual, pre)

    @staticmethod
    def backward(ctx, grad_out: torch.Tensor):
        residual, pre = ctx.saved_tensors
        grad_residual, grad_pre = h_aggregate_backward(residual, pre, grad_out.contiguous())
        return (grad_residual if ctx.needs_input_grad[0] else None,
                grad_pre if ctx.needs_input_grad[1] else None)


def h_aggregate_autograd(residual: torch.Tensor, pre: torch.Tensor) -> torch.Tensor:
    return HAggregate.apply(residual, pre)

"""Helpers for the GPU tests: run the library through its C ABI on cuda:0
with inputs from the shared generator, and bring raw bits back."""

from __future__ import annotations

import numpy as np
import torch

from hyper_connection_residual_mhc_amd import ops
from hyper_connection_residual_mhc_amd.workloads import (bf16_tensor_to_bits, bits_to_bf16_tensor,
                                                         to_device)

HC = 4
SPLIT, ROWS = 1, 2                 # backward layouts (MHC_BWD_SPLIT, MHC_BWD_ROWS)
SENTINELS = (0x7FC1, 0xFFEE)      # bf16 NaN patterns the kernels never produce
GUARD = 2048                       # elements of guard region on each side


def say(msg: str) -> None:
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(msg, flush=True)


def run_fwd(host: dict, dev, launch=None) -> np.ndarray:
    d = to_device({"residual": host["residual"], "pre": host["pre"]}, dev)
    T, _, H = host["residual"].shape
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ops.mhc_h_aggregate_fwd(d["residual"], d["pre"], out, launch=launch)
    torch.cuda.synchronize()
    return bf16_tensor_to_bits(out)


def run_bwd(host: dict, dev, launch=None) -> tuple[np.ndarray, np.ndarray]:
    d = to_device(host, dev)
    T, _, H = host["residual"].shape
    gr = torch.empty((T, HC, H), dtype=torch.bfloat16, device=dev)
    gp = torch.empty((T, HC), dtype=torch.float32, device=dev)
    ops.mhc_h_aggregate_bwd(d["residual"], d["pre"], d["grad_out"], gr, gp, launch=launch)
    torch.cuda.synchronize()
    return bf16_tensor_to_bits(gr), gp.cpu().numpy()


def guarded_empty_bf16(shape, dev, sentinel: int) -> tuple[torch.Tensor, torch.Tensor]:
    """A bf16 tensor of `shape` inside a larger buffer with GUARD elements on
    each side; the whole buffer is filled with `sentinel`. Returns (view, buffer)."""
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * GUARD,), sentinel, dtype=torch.int32, device=dev).to(torch.int16)
    view = buf[GUARD:GUARD + n].view(torch.bfloat16).view(shape)
    return view, buf


def guards_untouched(buf: torch.Tensor, n: int, sentinel: int) -> bool:
    b = buf.cpu().numpy().view(np.uint16)
    return bool((b[:GUARD] == sentinel).all() and (b[GUARD + n:] == sentinel).all())


def offset_copy_bf16(bits: np.ndarray, dev, offset_elems: int) -> torch.Tensor:
    """Device bf16 tensor with the given bits whose data pointer is
    `offset_elems` elements past a 256-byte-aligned allocation (to force
    narrower vector accesses)."""
    flat = bits.ravel()
    buf = torch.empty(flat.size + offset_elems, dtype=torch.bfloat16, device=dev)
    view = buf[offset_elems:].view(bits.shape)
    view.copy_(bits_to_bf16_tensor(bits, dev))
    return view


class HipEvents:
    """Raw timing events from the HIP runtime, for the *_timed entry points."""

    def __init__(self, n: int):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.h = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            self.h.append(e.value)

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = self.ct.c_float()
        assert self.hip.hipEventSynchronize(self.h[b]) == 0
        assert self.hip.hipEventElapsedTime(self.ct.byref(ms), self.h[a], self.h[b]) == 0
        return ms.value

    def close(self):
        for e in self.h:
            self.hip.hipEventDestroy(e)
        self.h = []

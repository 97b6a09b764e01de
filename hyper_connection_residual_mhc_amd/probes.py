"""Binding of the measurement library (csrc/mhc_probes.h): the device's bf16
rounding routine over a range of fp32 patterns, a byte stream with a given
read:write mix, and the same stream with per-wave clock stamps. Used by the
tests and the benchmark; not part of the operation. Argument marshalling
only, as in ops.py."""

from __future__ import annotations

import ctypes

import torch

from . import _lib


def _stream_handle(device: torch.device, stream: torch.cuda.Stream | None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return int(s.cuda_stream)


def mhc_bf16_rne_probe(first_bits: int, out: torch.Tensor,
                       stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """out[k] = device bf16 rounding of the fp32 pattern first_bits + k (out: int16/uint16)."""
    if out.device.type != "cuda" or out.dtype not in (torch.int16, torch.uint16, torch.bfloat16):
        raise TypeError("out must be a 16-bit GPU tensor")
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    with torch.cuda.device(out.device):
        st = _lib.probe_lib().mhc_bf16_rne_probe(int(first_bits) & 0xFFFFFFFF, out.numel(),
                                                 out.data_ptr(),
                                                 _stream_handle(out.device, stream))
    _lib.check_probe(st)
    return out


def mhc_stream_probe(src: torch.Tensor | None, dst: torch.Tensor | None, reads: int, writes: int,
                     stream: torch.cuda.Stream | None = None, start_event=None,
                     stop_event=None) -> torch.Tensor | None:
    """Per unit, read `reads` consecutive KiB of src and write `writes` KiB of
    dst with no arithmetic (mixes 1:1, 4:1, 5:4, 9:4, 8:0, 0:8; src is None
    for the write-only mix, dst None for the read-only one). Events are raw
    hipEvent_t handles or None."""
    dev = _probe_buffers(src, dst)
    ptr = lambda x: 0 if x is None else x.data_ptr()
    nbytes = lambda x: 0 if x is None else x.numel() * x.element_size()
    with torch.cuda.device(dev):
        st = _lib.probe_lib().mhc_stream_probe(ptr(src), nbytes(src), ptr(dst), nbytes(dst),
                                               int(reads), int(writes),
                                               _stream_handle(dev, stream), start_event,
                                               stop_event)
    _lib.check_probe(st)
    return dst


def _probe_buffers(src: torch.Tensor | None, dst: torch.Tensor | None) -> torch.device:
    dev = None
    for name, x in (("src", src), ("dst", dst)):
        if x is None:
            continue
        if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
            raise TypeError(f"{name} must be a GPU tensor or None")
        if not x.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        dev = x.device
    if dev is None:
        raise ValueError("src and dst cannot both be None")
    return dev


def mhc_clock_probe(src: torch.Tensor | None, dst: torch.Tensor | None, reads: int, writes: int,
                    waves_per_block: int, stamps: torch.Tensor,
                    stream: torch.cuda.Stream | None = None, start_event=None,
                    stop_event=None) -> torch.Tensor:
    """mhc_stream_probe's units with `waves_per_block` (1, 4, 16) units per
    block; stamps (int64 GPU tensor, at least 4 per unit) receives, per unit,
    the wall clock at the wave's start, after its loads, after its stores,
    and its XCD (low 32 bits) with its HW_ID register (high 32 bits)."""
    dev = _probe_buffers(src, dst)
    if (not isinstance(stamps, torch.Tensor) or stamps.device != dev
            or stamps.dtype != torch.int64 or not stamps.is_contiguous()):
        raise TypeError("stamps must be a contiguous int64 tensor on the buffers' GPU")
    ptr = lambda x: 0 if x is None else x.data_ptr()
    nbytes = lambda x: 0 if x is None else x.numel() * x.element_size()
    with torch.cuda.device(dev):
        st = _lib.probe_lib().mhc_clock_probe(ptr(src), nbytes(src), ptr(dst), nbytes(dst),
                                              int(reads), int(writes), int(waves_per_block),
                                              stamps.data_ptr(), stamps.numel(),
                                              _stream_handle(dev, stream), start_event,
                                              stop_event)
    _lib.check_probe(st)
    return stamps


def mhc_probe_wall_clock_khz(device: torch.device | int | None = None) -> int:
    """Rate of the wall clock the clock probe stamps with, in kHz."""
    khz = ctypes.c_int32()
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        _lib.check_probe(_lib.probe_lib().mhc_probe_wall_clock_khz(ctypes.byref(khz)))
    return int(khz.value)

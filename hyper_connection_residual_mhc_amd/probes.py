"""Binding of the measurement library (csrc/mhc_probes.h): the device's bf16
rounding routine over a range of fp32 patterns, and a byte stream with a
given read:write mix. Used by the tests and the benchmark; not part of the
operation. Argument marshalling only, as in ops.py."""

from __future__ import annotations

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
    ptr = lambda x: 0 if x is None else x.data_ptr()
    nbytes = lambda x: 0 if x is None else x.numel() * x.element_size()
    with torch.cuda.device(dev):
        st = _lib.probe_lib().mhc_stream_probe(ptr(src), nbytes(src), ptr(dst), nbytes(dst),
                                               int(reads), int(writes),
                                               _stream_handle(dev, stream), start_event,
                                               stop_event)
    _lib.check_probe(st)
    return dst

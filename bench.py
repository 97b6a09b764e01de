"""Benchmark of the mHC pre / H-aggregate hot path on one MI355X.

A step is one pass of the whole path on one batch: the forward
(residual[T,4,H], pre[T,4] -> out[T,H]) followed by the backward
(-> grad_residual[T,4,H], grad_pre[T,4]) at T=1024, H=7168, HC=4 - the
bandwidth shape of the page "Add batch-invariant h_aggregate kernel"
(RL-Kernel pull request 366), section Performance.

Cold caches: inputs and outputs rotate over `--sets` buffer sets (default 8,
about 1.2 GB) and the forward and backward of one step use different sets,
so every set's bytes leave the 256 MB Infinity Cache and the L2s before they
are touched again. Inputs are resident in HBM before anything is timed.

Timing, all on the stream the kernels are launched on:
* the timed region: `--steps` steps of plain launches, with a synchronize on
  both sides (host wall clock: `ms_per_step`, `value`) and two HIP events
  recorded on the stream around it (`step.gpu_us`);
* per-kernel time: blocks of back-to-back plain launches of one kernel on
  rotating cold sets, one event pair around each block of 100 launches
  after 10 untimed ones, 7 rounds (the protocol of the page "perf: fuse mHC
  coefficient backward epilogue", Performance Method); a round's figure is
  the block's time over its launch count, so every launch and the gaps
  between back-to-back dispatches are counted. `roofline` takes the
  backward's (the dominant kernel) median round;
* beside it, `dispatch_event_us`: the same kernel with HIP events attached
  to each dispatch itself (its start and end timestamps), for comparison;
* `shapes`: the forward and the backward at T=2048 and 8192 (H=7168) timed
  per call the same way, each with its fraction of the 8 TB/s peak;
* `stream_probes`: plain byte streams with the backward's 5:4 and the
  forward's 4:1 read:write mix, read only and write only, at the backward's
  bytes, timed the same way (the measurement library, not the operation);
* `cpu_baseline`: the CPU oracle on the same workload, on one core and on
  all cores, before the GPU is touched.

Output: one JSON line. `value` is the step's algorithmic bytes (forward
10H+16 and backward 18H+32 per token) divided by the measured time per step.
`roofline.traffic` comes from the committed counter summary while the
library's device code is the one it was measured on.

Helpers for the profiles: --summarize-stats and --summarize-pmc turn
rocprofv3 CSV output into the short text summaries kept in profiles/.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import platform
import re
import statistics
import struct
import subprocess
import sys
import time
from pathlib import Path

REPO = Path(__file__).resolve().parent
if str(REPO) not in sys.path:
    sys.path.insert(0, str(REPO))

METRIC = "h_aggregate fwd/bwd achieved HBM GB/s + µs/call at T=1024,H=7168 (1 GPU)"
HC = 4
PEAK_HBM_GBPS = 8000.0            # MI355X HBM3E peak, 8 TB/s
TRAFFIC_FILE = REPO / "profiles" / "hagg_bwd_T1024_H7168_traffic.md"


def fwd_bytes(T: int, H: int, n: int = HC) -> int:
    """Algorithmic bytes of one forward call: read residual (8H) and pre (16),
    write out (2H), per token (at expansion n: 2nH + 4n read, 2H written)."""
    return T * (2 * (n + 1) * H + 4 * n)


def bwd_bytes(T: int, H: int, n: int = HC) -> int:
    """Algorithmic bytes of one backward call: read residual (8H), grad_out
    (2H), pre (16); write grad_residual (8H), grad_pre (16), per token (at
    expansion n: (4n + 2)H + 8n)."""
    return T * ((4 * n + 2) * H + 8 * n)


def bwd_acc_bytes(T: int, H: int, n: int = HC) -> int:
    """Accumulating backward: the plain backward's bytes plus reading the
    stored grad_residual (8H; 2nH at expansion n) per token."""
    return T * ((6 * n + 2) * H + 8 * n)


def _elf_sections(blob: bytes) -> dict[str, bytes]:
    """Section name -> bytes of a little-endian ELF64 image."""
    shoff = struct.unpack_from("<Q", blob, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", blob, 0x3A)

    def header(i: int) -> tuple:
        return struct.unpack_from("<IIQQQQIIQQ", blob, shoff + i * shentsize)

    names = header(shstrndx)[4]
    out = {}
    for i in range(shnum):
        h = header(i)
        name = blob[names + h[0]:blob.index(b"\0", names + h[0])].decode()
        out[name] = blob[h[4]:h[4] + h[5]]
    return out


def device_code_sha256(lib_path: Path | None = None) -> str | None:
    """Digest of the gfx950 kernels in our built library: the machine code,
    kernel descriptors and kernel metadata (.text, .rodata, .note) of the
    gfx950 code object in its offload bundle. It changes exactly when a
    kernel changes (comments and host code leave it alone, and rebuilding
    the same source gives the same digest). None if there is no library."""
    from hyper_connection_residual_mhc_amd import _build
    path = lib_path or _build.LIB_PATH
    if not path.exists():
        return None
    bundle = _elf_sections(path.read_bytes()).get(".hip_fatbin")
    if not bundle or not bundle.startswith(b"__CLANG_OFFLOAD_BUNDLE__"):
        return None
    count = struct.unpack_from("<Q", bundle, 24)[0]
    pos = 32
    for _ in range(count):
        off, size, id_len = struct.unpack_from("<QQQ", bundle, pos)
        ident = bundle[pos + 24:pos + 24 + id_len].decode()
        pos += 24 + id_len
        if ident.endswith("gfx950"):
            sec = _elf_sections(bundle[off:off + size])
            h = hashlib.sha256()
            for name in (".text", ".rodata", ".note"):
                h.update(sec.get(name, b""))
            return h.hexdigest()
    return None


def recorded_traffic(T: int, H: int, kernel: str, text: str | None = None) -> int | None:
    """HBM bytes per backward launch from the committed counter summary, or
    None when there is none, when it covers another kernel or shape than the
    one timed (its title names both), or when the kernels changed since it
    was taken (device-code digest)."""
    if text is None:
        if not TRAFFIC_FILE.exists():
            return None
        text = TRAFFIC_FILE.read_text()
    title = text.splitlines()[0] if text else ""
    m_shape = re.search(r"\bT=(\d+), H=(\d+)\b", title)
    m_sha = re.search(r"device_code_sha256:\s*([0-9a-f]{64})", text)
    m_val = re.search(r"traffic_bytes_per_launch:\s*(\d+)", text)
    if not (m_shape and m_sha and m_val) or kernel not in title:
        return None
    if (int(m_shape.group(1)), int(m_shape.group(2))) != (T, H):
        return None
    if m_sha.group(1) != device_code_sha256():
        return None
    return int(m_val.group(1))


# ---------------------------------------------------------------------------
# GPU part
# ---------------------------------------------------------------------------

SEED = 0
BLOCK_TOKENS = 1024  # tokens drawn on the host; longer batches repeat them on the device


class BufferSet:
    """One independent set of device inputs and outputs for a step."""

    def __init__(self, d: dict, dev, hc: int = HC):
        import torch
        self.residual, self.pre, self.grad_out = d["residual"], d["pre"], d["grad_out"]
        T, _, H = self.residual.shape
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        self.grad_residual = torch.empty((T, hc, H), dtype=torch.bfloat16, device=dev)
        self.grad_pre = torch.empty((T, hc), dtype=torch.float32, device=dev)


def device_inputs(T: int, H: int, dev, hc: int = HC) -> dict:
    """Seeded inputs on the device: min(T, 1024) tokens drawn by the shared
    generator (seed 0, grad_out, 1% x64 residual outliers), repeated along
    the token axis up to T (the values only have to have the workload's
    distribution; drawing 8192 tokens on the host would take longer than
    the whole timed work)."""
    import torch
    from hyper_connection_residual_mhc_amd.workloads import make_inputs, to_device
    t0 = min(T, BLOCK_TOKENS)
    d = to_device(make_inputs(t0, H, seed=SEED, grad=True, outliers=True, hc=hc), dev)
    reps = -(-T // t0)
    if reps > 1:
        d = {k: v.repeat((reps,) + (1,) * (v.dim() - 1))[:T].contiguous() for k, v in d.items()}
    return d


def make_sets(T: int, H: int, n: int, dev, hc: int = HC) -> list[BufferSet]:
    """n sets with the same input values at different addresses (cold caches
    need distinct bytes in memory, not distinct values)."""
    src = device_inputs(T, H, dev, hc)
    sets = [BufferSet({k: v.clone() for k, v in src.items()}, dev, hc) for _ in range(n)]
    del src
    return sets


def copy_probe(dev, nbytes: int = 1 << 28, reps: int = 3) -> None:
    """A plain copy of known size, run outside the timed region so that
    counter runs can scale FETCH_SIZE / WRITE_SIZE: the measurement
    library's 1:1 stream (stream_probe_kernel<1, 1, 2>: reads nbytes, writes
    nbytes, nothing else), `reps` times."""
    import torch
    from hyper_connection_residual_mhc_amd import _lib
    plib = _lib.probe_lib()
    src = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    sh = int(torch.cuda.current_stream(dev).cuda_stream)
    for _ in range(reps):
        _lib.check_probe(plib.mhc_stream_probe(src.data_ptr(), nbytes, dst.data_ptr(), nbytes,
                                               1, 1, sh, None, None))
    torch.cuda.synchronize()


# Read:write mix of each kernel for the streaming probe (per token: forward
# 8H read / 2H written, backward 10H / 8H, accumulating backward 18H / 8H),
# and the read-only and write-only streams.
PROBE_MIX = {"fwd": (4, 1), "bwd": (5, 4), "bwd_acc": (9, 4), "read": (8, 0), "write": (0, 8)}


class ProbeBuffers:
    """Rotating src/dst pairs for mhc_stream_probe sized to about `nbytes`
    of traffic with the given mix (whole units of r + w KiB)."""

    def __init__(self, nbytes: int, mix: tuple[int, int], pairs: int, dev):
        import torch
        r, w = mix
        self.units = max(1, nbytes // ((r + w) * 1024))
        self.mix = mix
        self.bytes = self.units * (r + w) * 1024
        mk = lambda kib, fill: (torch.full((self.units * kib * 256,), fill, dtype=torch.int32,
                                           device=dev) if kib else None)
        self.pairs = [(mk(r, 1), mk(w, 0)) for _ in range(pairs)]

    def call(self, lib, k: int, stream_handle: int, a, b) -> int:
        src, dst = self.pairs[k % len(self.pairs)]
        r, w = self.mix
        ptr = lambda t: 0 if t is None else t.data_ptr()
        size = lambda t: 0 if t is None else t.numel() * 4
        return lib.mhc_stream_probe(ptr(src), size(src), ptr(dst), size(dst), r, w,
                                    stream_handle, a, b)


class HipEvents:
    """Timing events from the HIP runtime (created with timing enabled). The
    library attaches them to its kernel dispatches, so their elapsed time is
    the kernels' own execution time."""

    def __init__(self, n: int):
        import ctypes
        self._ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.handles = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.handles.append(h.value)

    def record(self, i: int, stream_handle: int) -> None:
        if self.hip.hipEventRecord(self.handles[i], stream_handle) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_us(self, a: int, b: int) -> float:
        ms = self._ct.c_float()
        if self.hip.hipEventElapsedTime(self._ct.byref(ms), self.handles[a], self.handles[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value * 1e3

    def close(self) -> None:
        for h in self.handles:
            self.hip.hipEventDestroy(h)
        self.handles = []


def round_stats(per_round: list[float]) -> dict:
    """Median and [p20, p50, p80] over per-round figures (any count >= 1)."""
    med = statistics.median(per_round)
    if len(per_round) >= 2:
        q = statistics.quantiles(per_round, n=10, method="inclusive")
        p20, p80 = q[1], q[7]
    else:
        p20 = p80 = med
    return {"us_median": round(med, 3), "us_p20_p50_p80": [round(p20, 3), round(med, 3),
                                                            round(p80, 3)],
            "rounds": len(per_round)}


class Timer:
    """Per-launch time of a callable fn(k, start_event, stop_event) -> status
    that launches one call on `stream_handle` (k picks the rotating set).

    block(fn): `rounds` rounds of `warm` untimed plain launches, then `timed`
    plain launches with one event pair recorded on the stream around them;
    a round's figure is the pair's elapsed time / `timed` (every launch, and
    the gaps between back-to-back dispatches, counted).
    dispatch(fn, n): n launches each carrying its own dispatch events (the
    dispatch's own start and end timestamps); per-launch microseconds.
    """

    def __init__(self, stream_handle: int, rounds: int = 7, warm: int = 10, timed: int = 100,
                 check=None):
        self.sh, self.rounds, self.warm, self.timed = stream_handle, rounds, warm, timed
        self.check = check
        self.ev = HipEvents(max(2, 2 * timed))

    def _ok(self, st: int) -> None:
        if st:
            self.check(st)

    def block(self, fn) -> list[float]:
        import torch
        out = []
        for _ in range(self.rounds):
            for k in range(self.warm):
                self._ok(fn(k, None, None))
            torch.cuda.synchronize()
            self.ev.record(0, self.sh)
            for k in range(self.timed):
                self._ok(fn(self.warm + k, None, None))
            self.ev.record(1, self.sh)
            torch.cuda.synchronize()
            out.append(self.ev.elapsed_us(0, 1) / self.timed)
        return out

    def dispatch(self, fn, n: int) -> list[float]:
        import torch
        n = min(n, self.timed)
        E = self.ev.handles
        for k in range(self.warm):
            self._ok(fn(k, None, None))
        torch.cuda.synchronize()
        for k in range(n):
            self._ok(fn(self.warm + k, E[2 * k], E[2 * k + 1]))
        torch.cuda.synchronize()
        return [self.ev.elapsed_us(2 * k, 2 * k + 1) for k in range(n)]

    def close(self) -> None:
        self.ev.close()


def kernel_record(nbytes: int, block: list[float], sampled: list[float] | None = None) -> dict:
    """Per-call figures of one kernel: block-timed median (all launches) with
    its GB/s and fraction of the HBM peak, plus the dispatch-event sample."""
    rec = {"bytes_per_call": nbytes, **round_stats(block)}
    med = rec["us_median"]
    rec["gbps"] = round(nbytes / med / 1e3, 1)
    rec["frac_of_8TBps"] = round(nbytes / med / 1e3 / PEAK_HBM_GBPS, 4)
    if sampled:
        rec["dispatch_event_us"] = {"launches": len(sampled),
                                    "mean": round(statistics.fmean(sampled), 3),
                                    "median": round(statistics.median(sampled), 3)}
    return rec


def _kernel_calls(lib, sets, T, H, sh):
    """fn(k, a, b) launchers of the forward and the backward on set k mod n."""
    nsets = len(sets)
    fargs = [(x.residual.data_ptr(), x.pre.data_ptr(), x.out.data_ptr(), T, H, sh) for x in sets]
    bargs = [(x.residual.data_ptr(), x.pre.data_ptr(), x.grad_out.data_ptr(),
              x.grad_residual.data_ptr(), x.grad_pre.data_ptr(), T, H, sh) for x in sets]

    def fwd(k, a, b):
        if a is None and b is None:
            return lib.mhc_h_aggregate_fwd(*fargs[k % nsets])
        return lib.mhc_h_aggregate_fwd_timed(*fargs[k % nsets], None, a, b)

    def bwd(k, a, b):
        if a is None and b is None:
            return lib.mhc_h_aggregate_bwd(*bargs[k % nsets])
        return lib.mhc_h_aggregate_bwd_timed(*bargs[k % nsets], None, a, b)
    return fwd, bwd


# Per-call shapes reported beside the step (H = 7168): (direction, T, sets).
SHAPES = [("fwd", 2048, 8), ("fwd", 8192, 3), ("bwd", 2048, 8), ("bwd", 8192, 3)]


def run_gpu(T: int, H: int, steps: int, warmup: int, nsets: int, copy_calibration: bool,
            sample: int = 32, shapes: bool = True, probes: bool = True) -> dict:
    """The timed forward + backward steps on nsets rotating cold buffer sets,
    then the per-kernel block timings (and dispatch-event samples) at the
    step's shape, at SHAPES and of the stream probes. copy_calibration:
    first run the plain device copy whose counter readings calibrate the
    traffic figures."""
    import torch
    from hyper_connection_residual_mhc_amd import _build, _lib, ops

    _build.ensure_built()
    lib = _lib.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sets = make_sets(T, H, nsets, dev)
    stream = torch.cuda.current_stream(dev)
    sh = int(stream.cuda_stream)

    s0 = sets[0]
    fwd_plan, fwd_grid = ops.mhc_h_aggregate_plan_fwd(s0.residual, s0.pre, s0.out, T, H)
    bwd_plan, bwd_grid = ops.mhc_h_aggregate_plan_bwd(s0.residual, s0.pre, s0.grad_out,
                                                      s0.grad_residual, s0.grad_pre, T, H)
    fwd, bwd = _kernel_calls(lib, sets, T, H, sh)

    if copy_calibration:
        copy_probe(dev)

    # Step k: forward on set 2k mod n, backward on set 2k+1 mod n.
    def step(k: int, a=None, b=None) -> int:
        return fwd(2 * k, None, None) | bwd(2 * k + 1, None, None)

    for k in range(warmup):
        st = step(k)
        if st:
            _lib.check(st)
    region = HipEvents(2)
    torch.cuda.synchronize()
    st = 0
    t0 = time.perf_counter()
    region.record(0, sh)
    for k in range(steps):
        st |= step(warmup + k)
    region.record(1, sh)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if st:
        _lib.check(st)
    region_us = region.elapsed_us(0, 1)
    region.close()

    tm = Timer(sh, check=_lib.check)
    out = {
        "wall_s": t1 - t0,
        "region_gpu_us": region_us,
        "step_block": tm.block(step),
        "fwd_block": tm.block(fwd),
        "bwd_block": tm.block(bwd),
        "fwd_sampled": tm.dispatch(fwd, sample) if sample else None,
        "bwd_sampled": tm.dispatch(bwd, sample) if sample else None,
        "fwd_plan": fwd_plan, "fwd_grid": fwd_grid,
        "bwd_plan": bwd_plan, "bwd_grid": bwd_grid,
        "device": torch.cuda.get_device_name(dev),
        "torch": torch.__version__,
        "hip": getattr(torch.version, "hip", None),
    }
    del sets, fwd, bwd
    torch.cuda.empty_cache()

    if probes:
        plib = _lib.probe_lib()
        out["probes"] = {}
        for name, nbytes in (("bwd", bwd_bytes(T, H)), ("fwd", fwd_bytes(T, H)),
                             ("read", bwd_bytes(T, H)), ("write", bwd_bytes(T, H))):
            pb = ProbeBuffers(nbytes, PROBE_MIX[name], nsets, dev)
            ptm = Timer(sh, check=_lib.check_probe)
            out["probes"][name] = {"bytes": pb.bytes,
                                   "block": ptm.block(lambda k, a, b: pb.call(plib, k, sh, a, b))}
            ptm.close()
            del pb
            torch.cuda.empty_cache()

    if shapes:
        out["shapes"] = []
        for direction, Ts, ns in SHAPES:
            ssets = make_sets(Ts, H, ns, dev)
            f, b = _kernel_calls(lib, ssets, Ts, H, sh)
            fn = f if direction == "fwd" else b
            out["shapes"].append({"direction": direction, "T": Ts, "H": H, "sets": ns,
                                  "block": tm.block(fn),
                                  "sampled": tm.dispatch(fn, sample) if sample else None})
            del ssets, f, b, fn
            torch.cuda.empty_cache()
    tm.close()
    return out


def probe_record(kernel_bytes: int, kernel_us: float, probe: dict, mix: str) -> dict:
    """A kernel against the plain stream with the given mix (block-timed medians)."""
    r, w = PROBE_MIX[mix]
    p = statistics.median(probe["block"])
    pg = probe["bytes"] / p / 1e3
    kg = kernel_bytes / kernel_us / 1e3
    return {"mix": f"{r}:{w}", "probe_bytes": probe["bytes"], "probe_us": round(p, 3),
            "probe_gbps": round(pg, 1), "kernel_us": round(kernel_us, 3),
            "kernel_gbps": round(kg, 1), "frac_of_probe": round(kg / pg, 4)}


def git_revision() -> str | None:
    """HEAD of the repository this file is in, or None where there is no
    git metadata (a copied tree)."""
    try:
        r = subprocess.run(["git", "-C", str(REPO), "rev-parse", "HEAD"], capture_output=True,
                           text=True, timeout=10)
        return r.stdout.strip() if r.returncode == 0 and r.stdout.strip() else None
    except (OSError, subprocess.SubprocessError):
        return None


def tree_digest() -> str:
    """sha256 over the files that define a run: the kernel sources and
    headers, the Python package and this file (name and content, sorted)."""
    files = sorted(list((REPO / "hyper_connection_residual_mhc_amd").glob("*.py")) +
                   list((REPO / "hyper_connection_residual_mhc_amd" / "csrc").glob("*")) +
                   list((REPO / "include").glob("*.h")) + [Path(__file__).resolve()])
    h = hashlib.sha256()
    for f in files:
        if f.is_file():
            h.update(f.relative_to(REPO).as_posix().encode() + b"\0" + f.read_bytes())
    return h.hexdigest()


# ---------------------------------------------------------------------------
# Shape sweep: per-call time of each kernel at the configured shapes
# ---------------------------------------------------------------------------

SWEEP_SHAPES = [  # (T, H): latency sweep, bandwidth shapes, backward shape
    (1, 4096), (8, 4096), (128, 4096), (1, 7168), (8, 7168), (128, 7168),
    (1024, 7168), (2048, 7168), (8192, 7168),
]
# (T, H, n): the other expansion rates at the bandwidth shapes
EXPANSION_SWEEP = [(1024, 7168, 2), (2048, 7168, 2), (1024, 7168, 8), (2048, 7168, 8)]
# (T, H, n): the row-layout backward's two issue priorities, written and
# accumulating, below, at and above one resident generation (T * n = 4,096
# rows on 256 CUs), and at other hidden sizes
PRIORITY_SWEEP = [(512, 7168, 4), (768, 7168, 4), (1024, 7168, 4), (1536, 7168, 4),
                  (2048, 7168, 4), (8192, 7168, 4), (2048, 7168, 2), (512, 7168, 8),
                  (1024, 2048, 4), (512, 4096, 4), (1024, 4096, 4), (1024, 8192, 4)]


class SweepTimer:
    """Per-call timing of the sweep: every timed launch carries its own
    dispatch events. `rounds` rounds; in each, every timed function runs in
    a block of its own: `warm` untimed launches, then `timed` timed ones,
    back to back."""

    def __init__(self, rounds: int, warm: int, timed: int):
        self.rounds, self.warm, self.timed = rounds, warm, timed
        self.ev = HipEvents(2 * timed)

    def blocks(self, fns, check) -> list[list[list[float]]]:
        """For each fn(k, start_event, stop_event) -> status, its per-round
        lists of microseconds. Within a round the functions run one after
        another, so neither inherits the other's write-back."""
        import torch
        E = self.ev.handles
        out = [[] for _ in fns]
        for _ in range(self.rounds):
            for fn, per_round in zip(fns, out):
                for k in range(self.warm):
                    check(fn(k, None, None))
                torch.cuda.synchronize()
                for k in range(self.timed):
                    check(fn(k, E[2 * k], E[2 * k + 1]))
                torch.cuda.synchronize()
                per_round.append([self.ev.elapsed_us(2 * k, 2 * k + 1) for k in range(self.timed)])
        return out

    @staticmethod
    def summary(per_round: list[list[float]]) -> tuple[float, list[float], float]:
        """Median of the round medians, [p20, p50, p80] over the round
        medians, and the mean of every launch."""
        med = [statistics.median(r) for r in per_round]
        rs = round_stats(med)
        mean = statistics.fmean([x for r in per_round for x in r])
        return statistics.median(med), rs["us_p20_p50_p80"], mean

    @classmethod
    def fields(cls, nbytes: int, per_round: list[list[float]]) -> dict:
        med, q, mean = cls.summary(per_round)
        return {"bytes": nbytes, "us_median": round(med, 3), "us_p20_p50_p80": q,
                "us_mean": round(mean, 3), "gbps": round(nbytes / med / 1e3, 1),
                "frac_of_8TBps": round(nbytes / med / 1e3 / PEAK_HBM_GBPS, 4)}

    def close(self) -> None:
        self.ev.close()


def wave_clock_summary(stamps, khz: int, dispatch_us: float | None = None) -> dict:
    """Where and when a launch's waves ran, from mhc_clock_probe's stamps
    ([units, 4]: start, loads returned, stores completed, XCD | HW_ID << 32).
    Times in us from the launch's first wave start; per XCD (by id): its first
    wave start, its last wave end, its wave count and median wave duration."""
    import numpy as np
    s = np.asarray(stamps, dtype=np.int64).reshape(-1, 4)
    us = 1000.0 / khz
    t0 = int(s[:, 0].min())
    xcc = s[:, 3] & 0xFFFFFFFF
    ids = sorted(int(x) for x in np.unique(xcc))
    first = [round((int(s[xcc == x, 0].min()) - t0) * us, 3) for x in ids]
    last = [round((int(s[xcc == x, 2].max()) - t0) * us, 3) for x in ids]
    rec = {"waves": int(s.shape[0]), "span_us": round((int(s[:, 2].max()) - t0) * us, 3),
           "xcd": ids, "xcd_waves": [int((xcc == x).sum()) for x in ids],
           "xcd_first_start_us": first, "xcd_last_end_us": last,
           "xcd_wave_us_median": [round(float(np.median(s[xcc == x, 2] - s[xcc == x, 0])) * us, 3)
                                  for x in ids],
           "start_stagger_us": round(max(first) - min(first), 3),
           "end_spread_us": round(max(last) - min(last), 3)}
    if dispatch_us is not None:
        rec["dispatch_us"] = round(dispatch_us, 3)
    return rec


def median_records(recs: list[dict]) -> dict:
    """Element-wise medians of wave_clock_summary records of one launch shape
    (lists by position; the XCD ids must agree)."""
    out = {}
    for k, v in recs[0].items():
        if k == "xcd":
            assert all(r["xcd"] == v for r in recs), "XCD ids differ between launches"
            out[k] = v
        elif isinstance(v, list):
            out[k] = [round(statistics.median(r[k][i] for r in recs), 3) for i in range(len(v))]
        else:
            out[k] = round(statistics.median(r[k] for r in recs), 3)
    return out


def run_wave_clock(path: str, T: int = 1024, H: int = 7168, reps: int = 5) -> None:
    """Per-wave clock stamps of the streaming probe at the bytes and read:write
    mix of the backward and of the forward at T, H, in blocks of 1, 4 and 16
    waves: how a launch's waves spread over the XCDs and over time, with no
    arithmetic in the way. Per shape, `reps` stamped launches that end a run
    of 10 back-to-back launches ("stream") and `reps` launched on an idle
    GPU ("alone"), each with its dispatch events; one JSON line per shape and
    mode with the element-wise medians over the reps."""
    import torch
    from hyper_connection_residual_mhc_amd import _build, _lib, probes

    _build.ensure_built()
    plib = _lib.probe_lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sh = int(torch.cuda.current_stream(dev).cuda_stream)
    khz = probes.mhc_probe_wall_clock_khz(dev)
    ev = HipEvents(2)
    ptr = lambda t: 0 if t is None else t.data_ptr()
    size = lambda t: 0 if t is None else t.numel() * 4
    with open(path, "w") as f:
        for name in ("bwd", "fwd"):
            nbytes = (bwd_bytes if name == "bwd" else fwd_bytes)(T, H)
            pb = ProbeBuffers(nbytes, PROBE_MIX[name], 8, dev)
            r, w = pb.mix
            stamps = torch.zeros(4 * pb.units, dtype=torch.int64, device=dev)
            for wpb in (1, 4, 16):
                def launch(k, a, b, wpb=wpb):
                    src, dst = pb.pairs[k % len(pb.pairs)]
                    _lib.check_probe(plib.mhc_clock_probe(
                        ptr(src), size(src), ptr(dst), size(dst), r, w, wpb, stamps.data_ptr(),
                        stamps.numel(), sh, a, b))
                for mode in ("stream", "alone"):
                    recs = []
                    for rep in range(reps):
                        for k in range(10):
                            launch(k, None, None)
                        if mode == "alone":
                            torch.cuda.synchronize()
                        launch(10 + rep, ev.handles[0], ev.handles[1])
                        torch.cuda.synchronize()
                        recs.append(wave_clock_summary(stamps.cpu().numpy(), khz,
                                                       ev.elapsed_us(0, 1)))
                    rec = {"probe": f"{r}:{w}", "like": name, "T": T, "H": H,
                           "bytes": pb.bytes, "units": pb.units, "waves_per_block": wpb,
                           "mode": mode, "reps": reps, "wall_clock_khz": khz,
                           **median_records(recs)}
                    f.write(json.dumps(rec) + "\n")
                    f.flush()
                    print(json.dumps(rec), flush=True)
            del pb, stamps
    ev.close()


def run_sweep(path: str, rounds: int = 7, warm: int = 10, timed: int = 100,
              part: str = "all") -> None:
    """Per-call forward and backward times at SWEEP_SHAPES, one JSON line per
    (shape, direction) into `path`. Every timed launch carries its own
    dispatch events, so launches run one at a time, each from cold caches
    (8 rotating buffer sets, 3 at T=8192) - the per-call latency a caller
    sees, as in the page's table. `rounds` rounds of `warm` untimed and
    `timed` timed launches; p20 / median / p80 are taken over the round
    medians, GB/s from the median. At T >= 1024 a streaming probe with the
    kernel's read:write byte mix is timed the same way in each round, in a
    block of its own after the kernel's (the reference column). Then the
    coefficient backward epilogue at COEFF_SWEEP, then forward, backward and
    accumulating backward at the other expansion rates (EXPANSION_SWEEP,
    through the *_n entry points, without probes), then the row-layout
    backward with each issue priority forced (PRIORITY_SWEEP, block-timed,
    the two alternating round by round). `part` limits the sweep to
    "h_aggregate", "coeff", "expansion" or "priority"."""
    import torch
    from hyper_connection_residual_mhc_amd import _build, _lib, ops

    _build.ensure_built()
    lib = _lib.lib()
    plib = _lib.probe_lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sh = int(torch.cuda.current_stream(dev).cuda_stream)
    tm = SweepTimer(rounds, warm, timed)
    blk = Timer(sh, rounds, warm, timed, check=_lib.check)

    def emit(f, rec: dict) -> None:
        f.write(json.dumps(rec) + "\n")
        f.flush()
        print(json.dumps(rec), file=sys.stderr, flush=True)

    with open(path, "w") as f:
        for T, H in (SWEEP_SHAPES if part in ("all", "h_aggregate") else []):
            nsets = 8 if T <= 2048 else 3
            sets = make_sets(T, H, nsets, dev)
            s0 = sets[0]
            directions = ("fwd", "bwd", "bwd_acc") if T >= 1024 else ("fwd", "bwd")
            for direction in directions:
                if direction == "fwd":
                    plan, _ = ops.mhc_h_aggregate_plan_fwd(s0.residual, s0.pre, s0.out, T, H)
                    nbytes = fwd_bytes(T, H)

                    def call(k, a, b):
                        x = sets[k % nsets]
                        return lib.mhc_h_aggregate_fwd_timed(
                            x.residual.data_ptr(), x.pre.data_ptr(), x.out.data_ptr(), T, H, sh,
                            None, a, b)
                elif direction == "bwd_acc":
                    plan, _ = ops.mhc_h_aggregate_plan_bwd_acc(s0.residual, s0.pre, s0.grad_out,
                                                               s0.grad_residual, s0.grad_pre, T, H)
                    nbytes = bwd_acc_bytes(T, H)

                    def call(k, a, b):
                        x = sets[k % nsets]
                        return lib.mhc_h_aggregate_bwd_acc(
                            x.residual.data_ptr(), x.pre.data_ptr(), x.grad_out.data_ptr(),
                            x.grad_residual.data_ptr(), x.grad_pre.data_ptr(), T, H, sh, None,
                            a, b)
                else:
                    plan, _ = ops.mhc_h_aggregate_plan_bwd(s0.residual, s0.pre, s0.grad_out,
                                                           s0.grad_residual, s0.grad_pre, T, H)
                    nbytes = bwd_bytes(T, H)

                    def call(k, a, b):
                        x = sets[k % nsets]
                        return lib.mhc_h_aggregate_bwd_timed(
                            x.residual.data_ptr(), x.pre.data_ptr(), x.grad_out.data_ptr(),
                            x.grad_residual.data_ptr(), x.grad_pre.data_ptr(), T, H, sh, None,
                            a, b)
                probe = (ProbeBuffers(nbytes, PROBE_MIX[direction], nsets, dev)
                         if T >= 1024 else None)
                fns = [call]
                if probe:
                    def probe_call(k, a, b, probe=probe):
                        _lib.check_probe(probe.call(plib, k, sh, a, b))
                        return 0
                    fns.append(probe_call)
                timings = tm.blocks(fns, _lib.check)
                rec = {"direction": direction, "T": T, "H": H,
                       **SweepTimer.fields(nbytes, timings[0]), "plan": plan,
                       "block": block_fields(nbytes, blk.block(call))}
                if probe:
                    pmed, _, _ = SweepTimer.summary(timings[1])
                    pg = probe.bytes / pmed / 1e3
                    rec["probe"] = {"mix": list(PROBE_MIX[direction]), "bytes": probe.bytes,
                                    "us_median": round(pmed, 3), "gbps": round(pg, 1),
                                    "frac_of_probe": round(rec["gbps"] / pg, 4)}
                    del probe
                emit(f, rec)
            del sets
            torch.cuda.empty_cache()
        for R, n, dtype in (COEFF_SWEEP if part in ("all", "coeff") else []):
            # the policy's form, then the two-launch form for comparison; the
            # oracle timed on the host beside the policy's fp32 form
            for launches in (0, 2):
                rec = time_coeff(R, n, dev, sh, tm, launches, dtype)
                if launches == 0 and dtype == "f32":
                    rec["cpu_baseline"] = run_coeff_cpu_baseline(R, n)
                emit(f, rec)
        for T, H, n in (EXPANSION_SWEEP if part in ("all", "expansion") else []):
            nsets = 8
            sets = make_sets(T, H, nsets, dev, hc=n)
            for direction in ("fwd", "bwd", "bwd_acc"):
                if direction == "fwd":
                    nbytes = fwd_bytes(T, H, n)

                    def call(k, a, b):
                        x = sets[k % nsets]
                        return lib.mhc_h_aggregate_fwd_n(
                            x.residual.data_ptr(), x.pre.data_ptr(), x.out.data_ptr(), T, n, H,
                            sh, None, a, b)
                else:
                    acc = int(direction == "bwd_acc")
                    nbytes = (bwd_acc_bytes if acc else bwd_bytes)(T, H, n)

                    def call(k, a, b, acc=acc):
                        x = sets[k % nsets]
                        return lib.mhc_h_aggregate_bwd_n(
                            x.residual.data_ptr(), x.pre.data_ptr(), x.grad_out.data_ptr(),
                            x.grad_residual.data_ptr(), x.grad_pre.data_ptr(), T, n, H, acc, sh,
                            None, a, b)
                timings = tm.blocks([call], _lib.check)
                emit(f, {"direction": direction, "T": T, "H": H, "n": n,
                         **SweepTimer.fields(nbytes, timings[0]),
                         "block": block_fields(nbytes, blk.block(call))})
            del sets
            torch.cuda.empty_cache()
        for T, H, n in (PRIORITY_SWEEP if part in ("all", "priority") else []):
            nsets = 8 if T <= 2048 else 3
            sets = make_sets(T, H, nsets, dev, hc=n)
            for acc in (0, 1):
                nbytes = (bwd_acc_bytes if acc else bwd_bytes)(T, H, n)
                s0 = sets[0]
                policy, _ = ops.mhc_h_aggregate_plan_bwd_n(s0.residual, s0.pre, s0.grad_out,
                                                           s0.grad_residual, s0.grad_pre, T, n,
                                                           H, accumulate=bool(acc))
                blocks = {}
                # FLAT and PROGRESS alternate round by round, so that both
                # see the same state of the GPU
                one = Timer(sh, 1, warm, timed, check=_lib.check)
                for _ in range(rounds):
                    for prio in (_lib.MHC_PRIO_FLAT, _lib.MHC_PRIO_PROGRESS):
                        launch = ops._launch_arg({"layout": _lib.MHC_BWD_ROWS,
                                                  "wave_priority": prio})

                        def call(k, a, b, acc=acc, launch=launch):
                            x = sets[k % nsets]
                            return lib.mhc_h_aggregate_bwd_n(
                                x.residual.data_ptr(), x.pre.data_ptr(), x.grad_out.data_ptr(),
                                x.grad_residual.data_ptr(), x.grad_pre.data_ptr(), T, n, H,
                                acc, sh, launch, a, b)
                        blocks.setdefault(prio, []).extend(one.block(call))
                one.close()
                flat = block_fields(nbytes, blocks[_lib.MHC_PRIO_FLAT])
                prog = block_fields(nbytes, blocks[_lib.MHC_PRIO_PROGRESS])
                emit(f, {"direction": "bwd_acc" if acc else "bwd", "T": T, "H": H, "n": n,
                         "bytes": nbytes, "policy_wave_priority": policy["wave_priority"],
                         "flat": flat, "progress": prog,
                         "progress_over_flat": round(prog["us_median"] / flat["us_median"], 4)})
            del sets
            torch.cuda.empty_cache()
    tm.close()
    blk.close()


def block_fields(nbytes: int, per_round: list[float]) -> dict:
    """Block-timed figures (every launch and dispatch gap counted)."""
    rs = round_stats(per_round)
    med = rs["us_median"]
    return {**rs, "gbps": round(nbytes / med / 1e3, 1),
            "frac_of_8TBps": round(nbytes / med / 1e3 / PEAK_HBM_GBPS, 4)}


# Launch shapes of the backward whose HBM traffic the counter runs compare
# (T=1024, H=7168): the policy's row layout with a token per block, the row
# layout with one row per block (a token's 4 waves in 4 blocks, which land on
# different XCDs and so different L2s), the split layout, and the row layout
# at half the vector width.
COUNTER_CASES = {
    "rows": {"layout": 2},
    "rows-1-per-block": {"layout": 2, "block_threads": 64},
    "split": {"layout": 1},
    "rows-v4": {"layout": 2, "vec_width": 4},
    "rows-flat": {"layout": 2, "wave_priority": 1},
    "rows-progress": {"layout": 2, "wave_priority": 2},
}
# And of the forward: the policy (one-wave blocks, 16-byte accesses), the
# page's 4-byte (bf16x2) accesses, and 1024-thread blocks.
FWD_COUNTER_CASES = {
    "fwd": {},
    "fwd-v2": {"vec_width": 2},
    "fwd-1024": {"block_threads": 1024},
}


def run_counter_case(case: str, T: int, H: int, launches: int = 64, nsets: int = 8) -> dict:
    """`launches` backward (or forward) calls in one launch shape on rotating cold sets
    (for rocprofv3 --pmc runs: FETCH_SIZE / WRITE_SIZE per dispatch), after
    the 256 MiB calibration copy. Returns the plan and the mean event time."""
    import torch
    from hyper_connection_residual_mhc_amd import _build, _lib, ops
    _build.ensure_built()
    lib = _lib.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sets = make_sets(T, H, nsets, dev)
    sh = int(torch.cuda.current_stream(dev).cuda_stream)
    forward = case in FWD_COUNTER_CASES
    shape = FWD_COUNTER_CASES[case] if forward else COUNTER_CASES[case]
    launch = ops._launch_arg(shape)
    s0 = sets[0]
    if forward:
        plan, grid = ops.mhc_h_aggregate_plan_fwd(s0.residual, s0.pre, s0.out, T, H,
                                                  launch=shape)
    else:
        plan, grid = ops.mhc_h_aggregate_plan_bwd(s0.residual, s0.pre, s0.grad_out,
                                                  s0.grad_residual, s0.grad_pre, T, H,
                                                  launch=shape)
    copy_probe(dev)
    ev = HipEvents(2 * launches)
    E = ev.handles
    for k in range(launches):
        x = sets[k % nsets]
        if forward:
            st = lib.mhc_h_aggregate_fwd_timed(x.residual.data_ptr(), x.pre.data_ptr(),
                                               x.out.data_ptr(), T, H, sh, launch,
                                               E[2 * k], E[2 * k + 1])
        else:
            st = lib.mhc_h_aggregate_bwd_timed(
                x.residual.data_ptr(), x.pre.data_ptr(), x.grad_out.data_ptr(),
                x.grad_residual.data_ptr(), x.grad_pre.data_ptr(), T, H, sh, launch,
                E[2 * k], E[2 * k + 1])
        _lib.check(st)
    torch.cuda.synchronize()
    us = statistics.fmean(ev.elapsed_us(2 * k, 2 * k + 1) for k in range(launches))
    ev.close()
    return {"case": case, "T": T, "H": H, "plan": plan, "grid_blocks": grid,
            "launches": launches, "us_mean": round(us, 3),
            "bytes": fwd_bytes(T, H) if forward else bwd_bytes(T, H)}


# The coefficient backward epilogue at the shapes of the page "perf: fuse
# mHC coefficient backward epilogue" (Performance Method: B = 4 sequences of
# T in {128, 512, 2048} tokens at HC = 4, so R = 4T rows; HC = 2 and 8 as
# controls at T = 512).
COEFF_SWEEP = [(512, 4, "f32"), (2048, 4, "f32"), (8192, 4, "f32"), (2048, 2, "f32"),
               (2048, 8, "f32"), (512, 4, "bf16"), (2048, 4, "bf16"), (8192, 4, "bf16")]
COEFF_KEYS = ("mix", "pre", "post", "grad_pre", "grad_post", "grad_res", "alpha")


def coeff_bytes(R: int, n: int, elem: int = 4) -> int:
    """Algorithmic bytes of one epilogue call with row tensors of `elem`
    bytes per value: per row mix, pre, post, grad_pre, grad_post, grad_res
    read and grad_mix written ((8n + 3n^2) values: 32n + 12n^2 bytes in
    fp32), plus alpha, grad_b and grad_alpha (fp32) once."""
    m = 2 * n + n * n
    return R * (8 * n + 3 * n * n) * elem + 12 + 4 * m + 12


def run_coeff_cpu_baseline(R: int, n: int, min_seconds: float = 1.0) -> dict:
    """The coefficient oracle, as it stands (numpy, one thread), on the same
    seed-0 inputs: calls repeated for at least `min_seconds` after one
    untimed call; microseconds per call."""
    from hyper_connection_residual_mhc_amd.workloads import make_coeff_inputs
    from oracle import coeff_bwd as CB
    host = make_coeff_inputs(R, n, seed=0)
    args = [host[k] for k in COEFF_KEYS]
    CB.coeff_bwd(*args, 2.0, n)
    calls, t0 = 0, time.perf_counter()
    while True:
        CB.coeff_bwd(*args, 2.0, n)
        calls += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": round(dt / calls * 1e6, 1), "unit": "us/call", "cores": 1, "kind": "oracle",
            "sample": f"{calls} calls of the oracle on the same {R}-row seed-0 inputs after one "
                      f"untimed call ({dt:.2f} s)"}


def time_coeff(R, n, dev, sh, tm: SweepTimer, launches=0, dtype: str = "f32") -> dict:
    """Per-call time of the coefficient epilogue (both of its launches,
    between the first dispatch's start and the last one's end) on row
    tensors stored as `dtype` (f32, bf16 or f16). Input sets rotate over
    more than the 256 MB Infinity Cache, so every call starts cold."""
    import torch
    from hyper_connection_residual_mhc_amd import _lib
    from hyper_connection_residual_mhc_amd.workloads import make_coeff_inputs
    clib = _lib.coeff_lib()
    fmt = {"f32": (_lib.MHC_COEFF_F32, torch.float32, 4),
           "bf16": (_lib.MHC_COEFF_BF16, torch.bfloat16, 2),
           "f16": (_lib.MHC_COEFF_F16, torch.float16, 2)}[dtype]
    host = make_coeff_inputs(R, n, seed=0)
    m = 2 * n + n * n
    per_set = coeff_bytes(R, n, fmt[2])
    nsets = max(8, min(4096, -(-(320 << 20) // per_set)))
    src = {k: torch.from_numpy(host[k]).to(dev) for k in COEFF_KEYS}
    src = {k: (v if k == "alpha" else v.to(fmt[1])) for k, v in src.items()}
    ws_bytes = clib.mhc_coeff_bwd_workspace_bytes(R, n)
    sets = []
    for _ in range(nsets):
        x = {k: v.clone() for k, v in src.items()}
        x["grad_mix"] = torch.empty((R, m), dtype=fmt[1], device=dev)
        x["grad_b"] = torch.empty((m,), dtype=torch.float32, device=dev)
        x["grad_alpha"] = torch.empty((3,), dtype=torch.float32, device=dev)
        x["ws"] = torch.zeros((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
        sets.append(x)

    def call(k, a, b):
        x = sets[k % nsets]
        return clib.mhc_coeff_bwd_ex(*(x[key].data_ptr() for key in COEFF_KEYS), 2.0,
                                     x["grad_mix"].data_ptr(), x["grad_b"].data_ptr(),
                                     x["grad_alpha"].data_ptr(), x["ws"].data_ptr(), ws_bytes, R,
                                     n, fmt[0], launches, sh, a, b)
    timings = tm.blocks([call], _lib.check_coeff)
    del sets, src
    torch.cuda.empty_cache()
    return {"op": "coeff_bwd", "rows": R, "n": n, "dtype": dtype, "sets": nsets,
            **SweepTimer.fields(per_set, timings[0]),
            "launches": clib.mhc_coeff_bwd_plan(R, n, launches), "chunks": -(-R // 64)}


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a token sample
# ---------------------------------------------------------------------------

def run_cpu_baseline(T: int, H: int, min_seconds: float) -> dict:
    """The oracle, as it stands, on the step's workload: the forward and
    backward of one seed-0 input set of T tokens, repeated until at least
    `min_seconds` of CPU time have passed (one thread: numpy ufuncs), after
    one untimed step."""
    from hyper_connection_residual_mhc_amd.workloads import make_inputs
    from oracle import h_aggregate as O
    host = make_inputs(T, H, seed=0, grad=True)
    # One untimed step first: the first call pays one-time costs (first
    # touch of fresh arrays), several seconds at this size.
    O.h_aggregate_fwd(host["residual"], host["pre"])
    O.h_aggregate_bwd(host["residual"], host["pre"], host["grad_out"])
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.h_aggregate_fwd(host["residual"], host["pre"])
        O.h_aggregate_bwd(host["residual"], host["pre"], host["grad_out"])
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= 1000:
            break
    gb = reps * (fwd_bytes(T, H) + bwd_bytes(T, H)) / 1e9
    return {
        "value": round(gb / dt, 6),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{reps} oracle steps (forward + backward) on one seed-0 input set of "
                   f"T={T}, H={H} (numpy float32 ufuncs, one thread) after one untimed step, {dt:.1f} s; "
                   f"GB/s of the same algorithmic bytes"),
        "host_cpu": cpu_model(),
        "host_cores_visible": len(os.sched_getaffinity(0)),
    }


_SLICES: list[dict] = []  # token slices handed to forked workers (inherited, not pickled)


def _oracle_worker(args: tuple[int, float]) -> tuple[int, float]:
    """Repeat the oracle's forward and backward on one token slice for at
    least `min_seconds`; return (repetitions, seconds)."""
    from oracle import h_aggregate as O
    i, min_seconds = args
    host = _SLICES[i]
    O.h_aggregate_fwd(host["residual"], host["pre"])  # untimed first step
    O.h_aggregate_bwd(host["residual"], host["pre"], host["grad_out"])
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.h_aggregate_fwd(host["residual"], host["pre"])
        O.h_aggregate_bwd(host["residual"], host["pre"], host["grad_out"])
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= 1000:
            return reps, dt


def run_cpu_baseline_all_cores(T: int, H: int, min_seconds: float, workers: int) -> dict:
    """The same oracle on every host core at once: tokens are independent,
    so the step's tokens are split into `workers` slices, one process each
    (forked before the GPU is touched). GB/s = all slices' algorithmic bytes
    over the slowest worker's time."""
    import multiprocessing as mp
    from hyper_connection_residual_mhc_amd.workloads import make_inputs
    host = make_inputs(T, H, seed=0, grad=True)
    bounds = [T * w // workers for w in range(workers + 1)]
    _SLICES.clear()
    _SLICES.extend({k: v[bounds[w]:bounds[w + 1]] for k, v in host.items()} for w in range(workers))
    with mp.get_context("fork").Pool(workers) as pool:
        res = pool.map(_oracle_worker, [(w, min_seconds) for w in range(workers)])
    _SLICES.clear()
    dt = max(t for _, t in res)
    nbytes = sum(r * (fwd_bytes(bounds[w + 1] - bounds[w], H) + bwd_bytes(bounds[w + 1] - bounds[w], H))
                 for w, (r, _) in enumerate(res))
    return {
        "value": round(nbytes / dt / 1e9, 6),
        "unit": "GB/s",
        "cores": workers,
        "kind": "oracle",
        "sample": (f"the T={T}, H={H} seed-0 step split into {workers} token slices, one "
                   f"process each, every slice's forward + backward repeated for at least "
                   f"{min_seconds:.0f} s ({min(r for r, _ in res)}-{max(r for r, _ in res)} "
                   f"repetitions); GB/s of the algorithmic bytes over the slowest worker's "
                   f"{dt:.1f} s"),
    }


def cpu_model() -> str:
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


# ---------------------------------------------------------------------------
# rocprofv3 summaries (for the text files in profiles/)
# ---------------------------------------------------------------------------

def _rows(path: str) -> list[dict]:
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _short_name(name: str) -> str:
    """Kernel name without return type, namespace or parameter list."""
    name = name.replace("(anonymous namespace)::", "")
    name = re.sub(r"^void ", "", name)
    return re.sub(r"\(.*", "", name)[:90]


def summarize_stats(path: str) -> None:
    """Markdown table of a rocprofv3 --stats kernel_stats.csv."""
    rows = _rows(path)
    print("| kernel | calls | avg us | min us | max us | total % |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        name = r.get("Name", "")
        short = _short_name(name)
        avg = float(r.get("AverageNs", 0)) / 1e3
        mn = float(r.get("MinNs", 0)) / 1e3
        mx = float(r.get("MaxNs", 0)) / 1e3
        print(f"| {short} | {r.get('Calls')} | {avg:.3f} | {mn:.3f} | {mx:.3f} | "
              f"{float(r.get('Percentage', 0)):.2f} |")


def summarize_db(path: str, match: str = "") -> None:
    """Markdown table of a rocprofv3 database (rocpd SQLite, the default
    output of ROCm 7): per kernel and grid size, the number of dispatches
    and the mean / median / min / max duration, for kernels whose name
    contains `match`."""
    import sqlite3
    con = sqlite3.connect(path)
    groups: dict[tuple[str, int, int, int], list[float]] = {}
    for name, gx, gy, wx, dur in con.execute(
            "select name, grid_x, grid_y, workgroup_x, duration from kernels"):
        if match and match not in name:
            continue
        groups.setdefault((_short_name(name), gx, gy, wx), []).append(dur / 1e3)
    con.close()
    print("| kernel | grid (work-items x, y) | block | dispatches | mean us | median us | "
          "min us | max us |")
    print("|---|---|---|---|---|---|---|---|")
    for (name, gx, gy, wx), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        print(f"| {name} | {gx} x {gy} | {wx} | {len(v)} | {statistics.fmean(v):.3f} | "
              f"{statistics.median(v):.3f} | {min(v):.3f} | {max(v):.3f} |")


def summarize_pmc(paths: list[str]) -> None:
    """Per-kernel average of each counter (KiB for FETCH_SIZE / WRITE_SIZE)
    from rocprofv3 --pmc counter_collection.csv files, one row per kernel and
    grid size (so the calibration copy stands apart from small staging copies)."""
    acc: dict[tuple[str, int, str], list[float]] = {}
    for p in paths:
        for r in _rows(p):
            key = (_short_name(r.get("Kernel_Name", "")), int(r.get("Grid_Size", 0) or 0),
                   r.get("Counter_Name", ""))
            acc.setdefault(key, []).append(float(r.get("Counter_Value", 0)))
    print("| kernel | grid size | counter | dispatches | average per dispatch |")
    print("|---|---|---|---|---|")
    for (name, grid, ctr), vals in sorted(acc.items()):
        print(f"| {name} | {grid} | {ctr} | {len(vals)} | {statistics.fmean(vals):.1f} |")


# ---------------------------------------------------------------------------

def build_record(args, g: dict, cpu: dict | None) -> dict:
    """The JSON line from run_gpu's measurements (no GPU needed here)."""
    T, H = args.tokens, args.hidden
    ms_per_step = g["wall_s"] * 1e3 / args.steps
    step_bytes = fwd_bytes(T, H) + bwd_bytes(T, H)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    fwd = kernel_record(fwd_bytes(T, H), g["fwd_block"], g.get("fwd_sampled"))
    bwd = kernel_record(bwd_bytes(T, H), g["bwd_block"], g.get("bwd_sampled"))
    fwd.update(plan=g["fwd_plan"], grid_blocks=g["fwd_grid"])
    bwd.update(plan=g["bwd_plan"], grid_blocks=g["bwd_grid"])
    step_block = round_stats(g["step_block"])
    bwd_us = bwd["us_median"]
    achieved = bwd_bytes(T, H) / (bwd_us * 1e-6) / 1e9
    bwd_kernel = ("hagg_bwd_rows_kernel" if g["bwd_plan"].get("layout") == 2 else
                  "hagg_bwd_kernel")
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"h_aggregate forward+backward, T={T}, H={H}, HC=4, bf16 in/out, "
                        f"fp32 pre and arithmetic",
            "T": T, "H": H, "hc": HC,
            "rotating_sets": args.sets,
            "bytes_per_step": step_bytes,
            "seed": SEED,
            "inputs": f"seed-{SEED} draws of the shared generator (residual N(0,1) with 1% x64 "
                      f"outliers, pre U[0,1), grad_out N(0,0.1)), {BLOCK_TOKENS}-token blocks "
                      f"repeated for longer batches; the same values in every rotating set",
        },
        "step": {"wall_us": round(ms_per_step * 1e3, 3),
                 "gpu_us": round(g["region_gpu_us"] / args.steps, 3),
                 "block": step_block,
                 "fwd_plus_bwd_block_us": round(fwd["us_median"] + bwd_us, 3)},
        "fwd": fwd,
        "bwd": bwd,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": recorded_traffic(T, H, bwd_kernel),
            "kernel": bwd_kernel + (" (backward, row layout)" if bwd_kernel == "hagg_bwd_rows_kernel"
                                    else " (backward, split layout)"),
            "timing": "median over 7 rounds of one event pair around 100 back-to-back plain "
                      "launches on rotating cold sets (every launch and dispatch gap counted)",
        },
        "timing": {"per_step": "host wall clock over the timed steps, synchronized on both "
                               "sides; step.gpu_us from HIP events recorded on the stream "
                               "around the same region",
                   "per_kernel": "blocks of back-to-back plain launches (7 rounds x (10 + 100)), "
                                 "one event pair per block on the kernels' stream; "
                                 "dispatch_event_us: events attached to each dispatch"},
        "device": g["device"],
        "torch": g["torch"],
        "hip": g["hip"],
        "git_sha": git_revision(),
        "tree_sha256": tree_digest(),
        "device_code_sha256": device_code_sha256(),
    }
    if g.get("probes"):
        pr = g["probes"]
        line["stream_probes"] = {
            "bwd": probe_record(bwd_bytes(T, H), bwd_us, pr["bwd"], "bwd"),
            "fwd": probe_record(fwd_bytes(T, H), fwd["us_median"], pr["fwd"], "fwd"),
            "read_only": probe_record(bwd_bytes(T, H), bwd_us, pr["read"], "read"),
            "write_only": probe_record(bwd_bytes(T, H), bwd_us, pr["write"], "write"),
        }
    if g.get("shapes"):
        line["shapes"] = []
        for sh in g["shapes"]:
            nb = (fwd_bytes if sh["direction"] == "fwd" else bwd_bytes)(sh["T"], sh["H"])
            line["shapes"].append({"direction": sh["direction"], "T": sh["T"], "H": sh["H"],
                                   "rotating_sets": sh["sets"],
                                   **kernel_record(nb, sh["block"], sh.get("sampled"))})
    if cpu is not None:
        line["cpu_baseline"] = cpu
    return line


def main(argv: list[str] | None = None, gpu_runner=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--sets", type=int, default=8, help="rotating buffer sets (cold caches)")
    ap.add_argument("--tokens", type=int, default=1024)
    ap.add_argument("--hidden", type=int, default=7168)
    ap.add_argument("--sample", type=int, default=32,
                    help="launches of each kernel timed by per-dispatch events (0: none)")
    ap.add_argument("--no-shapes", action="store_true", help="skip the T=2048/8192 figures")
    ap.add_argument("--no-probes", action="store_true", help="skip the stream probes")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run a 256 MiB device copy first (counter calibration)")
    ap.add_argument("--sweep", metavar="OUT_JSONL",
                    help="instead of the step benchmark, time each kernel per call at the "
                         "latency / bandwidth / backward shapes and write JSON lines")
    ap.add_argument("--sweep-part",
                    choices=("all", "h_aggregate", "coeff", "expansion", "priority"),
                    default="all",
                    help="with --sweep: which operations to time")
    ap.add_argument("--wave-clock", metavar="OUT_JSONL",
                    help="instead of the step benchmark, stamp the streaming probe's waves at "
                         "the kernels' bytes (where and when each wave ran) and write JSON lines")
    ap.add_argument("--counter-case", choices=sorted(COUNTER_CASES) + sorted(FWD_COUNTER_CASES),
                    help="instead of the step benchmark, run 64 backward (or forward) calls in "
                         "one launch shape (for rocprofv3 --pmc runs) and print one JSON line")
    ap.add_argument("--summarize-stats", metavar="KERNEL_STATS_CSV")
    ap.add_argument("--summarize-pmc", metavar="COUNTER_CSV", nargs="+")
    ap.add_argument("--summarize-db", metavar="ROCPD_DB",
                    help="per-kernel, per-grid durations from a rocprofv3 database")
    ap.add_argument("--match", default="", help="with --summarize-db: kernel name filter")
    args = ap.parse_args(argv)

    if args.summarize_db:
        summarize_db(args.summarize_db, args.match)
        return 0
    if args.summarize_stats:
        summarize_stats(args.summarize_stats)
        return 0
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return 0
    if args.counter_case:
        print(json.dumps(run_counter_case(args.counter_case, args.tokens, args.hidden,
                                          nsets=args.sets)))
        return 0
    if args.wave_clock:
        if args.gpus != 1:
            print("the wave clock runs on one GPU", file=sys.stderr)
            return 2
        run_wave_clock(args.wave_clock, args.tokens, args.hidden)
        return 0
    if args.sweep:
        if args.gpus != 1:
            print("the sweep runs on one GPU", file=sys.stderr)
            return 2
        run_sweep(args.sweep, part=args.sweep_part)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this operation is token-parallel with no "
              f"communication, and runs here on a single MI355X (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2
    if args.sets < 2:
        print("--sets must be >= 2 (forward and backward use different sets)", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0 or args.sample < 0:
        print("--steps must be >= 1, --warmup and --sample >= 0", file=sys.stderr)
        return 2

    T, H = args.tokens, args.hidden
    # The oracle baselines run first, before anything touches the GPU (the
    # all-core one forks worker processes).
    cpu = None
    if not args.no_cpu_baseline:
        cpu = run_cpu_baseline(T, H, args.cpu_seconds)
        workers = min(16, len(os.sched_getaffinity(0)))
        if workers > 1:
            cpu["all_cores"] = run_cpu_baseline_all_cores(T, H, args.cpu_seconds, workers)
    runner = gpu_runner or run_gpu
    g = runner(T, H, args.steps, args.warmup, args.sets, args.copy_probe, sample=args.sample,
               shapes=not args.no_shapes, probes=not args.no_probes)
    print(json.dumps(build_record(args, g, cpu)), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

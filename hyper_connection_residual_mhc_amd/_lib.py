"""ctypes view of the C ABIs in include/mhc_h_aggregate.h and
include/mhc_coeff_bwd.h, and of the measurement library (csrc/mhc_probes.h)
that the tests and the benchmark use.

Loading fails loudly (ImportError) when a shared library has not been built,
or was built from other sources than the ones in the tree (the digest
recorded beside it at build time no longer matches): there is no other
implementation to fall back on, and a stale binary is never run by mistake.
"""

from __future__ import annotations

import ctypes
from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_int64, c_uint32, c_void_p

from . import _build
from ._build import COEFF_LIB_PATH, COEFF_SRC, LIB_PATH, PROBE_LIB_PATH, PROBE_SRC, SRC

MHC_SUCCESS = 0
MHC_ERROR_INVALID_VALUE = 1
MHC_ERROR_ALIASING = 2
MHC_ERROR_HIP = 3
MHC_ABI_VERSION = 5
MHC_BWD_SPLIT = 1
MHC_BWD_ROWS = 2
MHC_PRIO_FLAT = 1
MHC_PRIO_PROGRESS = 2
MHC_MAX_H = 1 << 26


class mhc_launch(ctypes.Structure):
    """Launch shape (see the header): 0 in a field means "policy chooses"."""
    _fields_ = [
        ("block_threads", c_int32),
        ("vec_width", c_int32),
        ("units_per_thread", c_int32),
        ("tokens_per_block", c_int32),
        ("streams_per_block", c_int32),
        ("layout", c_int32),
        ("wave_priority", c_int32),
    ]

    def as_dict(self) -> dict:
        return {name: int(getattr(self, name)) for name, _ in self._fields_}


# name -> (restype, argtypes); every symbol the header declares.
SIGNATURES = {
    "mhc_abi_version": (c_int, []),
    "mhc_status_string": (c_char_p, [c_int]),
    "mhc_last_error_message": (c_char_p, []),
    "mhc_h_aggregate_fwd": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_void_p]),
    "mhc_h_aggregate_fwd_ex": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_void_p,
                                       POINTER(mhc_launch)]),
    "mhc_h_aggregate_bwd": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_int64, c_int64, c_void_p]),
    "mhc_h_aggregate_bwd_ex": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_int64, c_int64, c_void_p, POINTER(mhc_launch)]),
    "mhc_h_aggregate_fwd_timed": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64,
                                          c_void_p, POINTER(mhc_launch), c_void_p, c_void_p]),
    "mhc_h_aggregate_bwd_timed": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_int64, c_int64, c_void_p, POINTER(mhc_launch),
                                          c_void_p, c_void_p]),
    "mhc_h_aggregate_bwd_acc": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_int64, c_int64, c_void_p, POINTER(mhc_launch),
                                        c_void_p, c_void_p]),
    "mhc_h_aggregate_plan_bwd_acc": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                             c_int64, c_int64, POINTER(mhc_launch),
                                             POINTER(mhc_launch), POINTER(c_int64)]),
    "mhc_h_aggregate_fwd_n": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int32, c_int64,
                                      c_void_p, POINTER(mhc_launch), c_void_p, c_void_p]),
    "mhc_h_aggregate_bwd_n": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_int64, c_int32, c_int64, c_int32, c_void_p,
                                      POINTER(mhc_launch), c_void_p, c_void_p]),
    "mhc_h_aggregate_plan_fwd_n": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int32,
                                           c_int64, POINTER(mhc_launch), POINTER(mhc_launch),
                                           POINTER(c_int64)]),
    "mhc_h_aggregate_plan_bwd_n": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                           c_int64, c_int32, c_int64, c_int32,
                                           POINTER(mhc_launch), POINTER(mhc_launch),
                                           POINTER(c_int64)]),
    "mhc_h_aggregate_validate_fwd": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64]),
    "mhc_h_aggregate_validate_bwd": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                             c_int64, c_int64]),
    "mhc_h_aggregate_plan_fwd": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64,
                                         POINTER(mhc_launch), POINTER(mhc_launch),
                                         POINTER(c_int64)]),
    "mhc_h_aggregate_plan_bwd": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_int64, c_int64, POINTER(mhc_launch),
                                         POINTER(mhc_launch), POINTER(c_int64)]),
}

MHC_COEFF_ABI_VERSION = 4
MHC_COEFF_CHUNK = 64
MHC_COEFF_MAX_ROWS = 1 << 28

# Every symbol include/mhc_coeff_bwd.h declares.
COEFF_SIGNATURES = {
    "mhc_coeff_abi_version": (c_int, []),
    "mhc_coeff_last_error_message": (c_char_p, []),
    "mhc_coeff_bwd_workspace_bytes": (c_int64, [c_int64, c_int32]),
    "mhc_coeff_bwd_plan": (c_int32, [c_int64, c_int32, c_int32]),
    "mhc_coeff_bwd_validate": (c_int, [c_void_p] * 7 + [c_float] + [c_void_p] * 4
                               + [c_int64, c_int64, c_int32]),
    "mhc_coeff_bwd": (c_int, [c_void_p] * 7 + [c_float] + [c_void_p] * 4
                      + [c_int64, c_int64, c_int32, c_int32, c_void_p, c_void_p, c_void_p]),
    "mhc_coeff_bwd_noalloc": (c_int, [c_void_p] * 7 + [c_float] + [c_void_p] * 3
                              + [c_int64, c_int32, c_int32, c_void_p, c_void_p, c_void_p]),
    "mhc_coeff_bwd_validate_ex": (c_int, [c_void_p] * 7 + [c_float] + [c_void_p] * 4
                                  + [c_int64, c_int64, c_int32, c_int32]),
    "mhc_coeff_bwd_ex": (c_int, [c_void_p] * 7 + [c_float] + [c_void_p] * 4
                         + [c_int64, c_int64, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                            c_void_p]),
}
MHC_COEFF_F32, MHC_COEFF_BF16, MHC_COEFF_F16 = 0, 1, 2
MHC_COEFF_SCRATCH_BYTES = 2 << 20

MHC_PROBE_ABI_VERSION = 2

# Every symbol csrc/mhc_probes.h declares.
PROBE_SIGNATURES = {
    "mhc_probe_abi_version": (c_int, []),
    "mhc_probe_last_error_message": (c_char_p, []),
    "mhc_bf16_rne_probe": (c_int, [c_uint32, c_int64, c_void_p, c_void_p]),
    "mhc_stream_probe": (c_int, [c_void_p, c_int64, c_void_p, c_int64, c_int32, c_int32,
                                 c_void_p, c_void_p, c_void_p]),
    "mhc_clock_probe": (c_int, [c_void_p, c_int64, c_void_p, c_int64, c_int32, c_int32, c_int32,
                                c_void_p, c_int64, c_void_p, c_void_p, c_void_p]),
    "mhc_probe_wall_clock_khz": (c_int, [POINTER(c_int32)]),
}

_loaded: dict[str, ctypes.CDLL] = {}


def open_checked(path, src, signatures: dict, version_fn: str, version: int) -> ctypes.CDLL:
    """Load the library at `path` after checking that it exists and that the
    digest recorded beside it matches `src` and the headers now in the tree;
    declare every signature and check the ABI version. ImportError otherwise."""
    if not path.exists():
        raise ImportError(f"{path} is missing: build it with __graft_entry__.build() "
                          "(the operation has no other implementation)")
    want = _build.source_digest(src)
    have = _build.recorded_digest(path)
    if have != want:
        raise ImportError(f"{path} was built from other sources than the ones in the tree "
                          f"(recorded digest {str(have)[:16]}, sources {want[:16]}): rebuild it "
                          "with __graft_entry__.build()")
    handle = ctypes.CDLL(str(path))
    for name, (restype, argtypes) in signatures.items():
        fn = getattr(handle, name)
        fn.restype = restype
        fn.argtypes = argtypes
    if getattr(handle, version_fn)() != version:
        raise ImportError(f"{path.name}: ABI version mismatch")
    return handle


def _get(key: str, *args) -> ctypes.CDLL:
    if key not in _loaded:
        _loaded[key] = open_checked(*args)
    return _loaded[key]


def lib() -> ctypes.CDLL:
    """The h_aggregate library (loaded once). ImportError if missing or stale."""
    return _get("h_aggregate", LIB_PATH, SRC, SIGNATURES, "mhc_abi_version", MHC_ABI_VERSION)


def coeff_lib() -> ctypes.CDLL:
    """The coefficient-backward library (loaded once). ImportError if missing
    or stale."""
    return _get("coeff", COEFF_LIB_PATH, COEFF_SRC, COEFF_SIGNATURES, "mhc_coeff_abi_version",
                MHC_COEFF_ABI_VERSION)


def probe_lib() -> ctypes.CDLL:
    """The measurement library (loaded once). ImportError if missing or stale."""
    return _get("probes", PROBE_LIB_PATH, PROBE_SRC, PROBE_SIGNATURES, "mhc_probe_abi_version",
                MHC_PROBE_ABI_VERSION)


class MhcError(RuntimeError):
    """A non-success status from the library, with its message."""

    def __init__(self, status: int, message: str):
        self.status = status
        name = lib().mhc_status_string(status).decode()
        super().__init__(f"{name}: {message}")


def check(status: int) -> None:
    if status != MHC_SUCCESS:
        raise MhcError(status, lib().mhc_last_error_message().decode())


def check_coeff(status: int) -> None:
    if status != MHC_SUCCESS:
        raise MhcError(status, coeff_lib().mhc_coeff_last_error_message().decode())


def check_probe(status: int) -> None:
    if status != MHC_SUCCESS:
        raise MhcError(status, probe_lib().mhc_probe_last_error_message().decode())

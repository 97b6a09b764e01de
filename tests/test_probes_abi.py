"""The measurement library on the host (csrc/mhc_probes.h): it exports what
its header declares and nothing of the operation, and the argument rules
hold before any HIP call (no GPU needed)."""

from __future__ import annotations

import re
import subprocess

import pytest

from hyper_connection_residual_mhc_amd import _build, _lib
from hyper_connection_residual_mhc_amd._lib import (MHC_ERROR_ALIASING, MHC_ERROR_INVALID_VALUE,
                                                    MHC_SUCCESS)

HEADER = _build.PKG_DIR / "csrc" / "mhc_probes.h"
GiB = 1 << 30
BASE = 16 * GiB
KiB = 1024


@pytest.fixture(scope="module")
def lib(built_library):
    return _lib.probe_lib()


def test_header_declarations_are_all_exported(lib):
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    names = sorted(set(re.findall(r"\b(mhc_\w+)\s*\(", text)))
    out = subprocess.run(["nm", "-D", "--defined-only", str(_build.PROBE_LIB_PATH)],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (mhc_\w+)$", out, flags=re.M))
    assert set(names) == exported == set(_lib.PROBE_SIGNATURES)
    assert lib.mhc_probe_abi_version() == _lib.MHC_PROBE_ABI_VERSION


def test_operation_library_no_longer_exports_the_probes(built_library):
    out = subprocess.run(["nm", "-D", "--defined-only", str(built_library)],
                         capture_output=True, text=True, check=True).stdout
    assert "probe" not in out


def test_rounding_probe_rejects_bad_sizes(lib):
    assert lib.mhc_bf16_rne_probe(0, -1, 1024, None) == MHC_ERROR_INVALID_VALUE
    assert lib.mhc_bf16_rne_probe(0, (1 << 32) + 1, 1024, None) == MHC_ERROR_INVALID_VALUE
    assert lib.mhc_bf16_rne_probe(0, 0, 0, None) == MHC_SUCCESS
    assert lib.mhc_bf16_rne_probe(0, 16, 0, None) == MHC_ERROR_INVALID_VALUE
    assert lib.mhc_bf16_rne_probe(0, 16, 1025, None) == MHC_ERROR_INVALID_VALUE
    assert b"aligned" in lib.mhc_probe_last_error_message()


def test_stream_probe_rejects_bad_arguments_before_any_hip_call(lib):
    src, dst = BASE, BASE + GiB
    probe = lib.mhc_stream_probe
    for reads, writes in ((2, 1), (5, 5), (0, 1), (4, 4), (-5, 4), (8, 1), (1, 8), (0, 0)):
        assert probe(src, 20 * KiB, dst, 16 * KiB, reads, writes, None, None,
                     None) == MHC_ERROR_INVALID_VALUE, (reads, writes)
    assert probe(src, 5 * KiB + 16, dst, 4 * KiB, 5, 4, None, None, None) == MHC_ERROR_INVALID_VALUE
    assert probe(src, 10 * KiB, dst, 4 * KiB, 5, 4, None, None, None) == MHC_ERROR_INVALID_VALUE
    assert probe(src, -5 * KiB, dst, 4 * KiB, 5, 4, None, None, None) == MHC_ERROR_INVALID_VALUE
    assert probe(src, 10 * KiB, src + 4 * KiB, 8 * KiB, 5, 4, None, None,
                 None) == MHC_ERROR_ALIASING
    assert probe(src + 8, 5 * KiB, dst, 4 * KiB, 5, 4, None, None, None) == MHC_ERROR_INVALID_VALUE
    assert probe(0, 0, 0, 0, 9, 4, None, None, None) == MHC_SUCCESS
    # read only: dst must be empty; write only: src must be empty
    assert probe(src, 16 * KiB, dst, 4 * KiB, 8, 0, None, None, None) == MHC_ERROR_INVALID_VALUE
    assert probe(src + 4, 16 * KiB, 0, 0, 8, 0, None, None, None) == MHC_ERROR_INVALID_VALUE
    assert probe(src, 4 * KiB, dst, 16 * KiB, 0, 8, None, None, None) == MHC_ERROR_INVALID_VALUE
    assert probe(0, 0, dst, 12 * KiB, 0, 8, None, None, None) == MHC_ERROR_INVALID_VALUE
    assert probe(0, 0, dst + 8, 16 * KiB, 0, 8, None, None, None) == MHC_ERROR_INVALID_VALUE
    assert probe(0, 0, 0, 0, 0, 8, None, None, None) == MHC_SUCCESS


def test_clock_probe_rejects_bad_arguments_before_any_hip_call(lib):
    src, dst, st = BASE, BASE + GiB, BASE + 2 * GiB
    probe = lib.mhc_clock_probe
    # 10 units of the 5:4 mix need 40 stamps
    good = (src, 50 * KiB, dst, 40 * KiB, 5, 4)
    for wpb in (0, 2, 3, 8, 32, -4):
        assert probe(*good, wpb, st, 40, None, None, None) == MHC_ERROR_INVALID_VALUE, wpb
    assert probe(*good, 4, st, 39, None, None, None) == MHC_ERROR_INVALID_VALUE
    assert b"stamps" in lib.mhc_probe_last_error_message()
    assert probe(*good, 4, st + 4, 40, None, None, None) == MHC_ERROR_INVALID_VALUE
    assert probe(*good, 4, 0, 40, None, None, None) == MHC_ERROR_INVALID_VALUE
    assert probe(*good, 4, src + 8 * KiB, 40, None, None, None) == MHC_ERROR_ALIASING
    assert probe(*good, 4, dst + 39 * KiB, 40, None, None, None) == MHC_ERROR_ALIASING
    # the stream probe's own rules apply
    assert probe(src, 50 * KiB, dst, 40 * KiB, 5, 5, 4, st, 40, None, None,
                 None) == MHC_ERROR_INVALID_VALUE
    assert probe(src, 50 * KiB, src + 16 * KiB, 40 * KiB, 5, 4, 4, st, 40, None, None,
                 None) == MHC_ERROR_ALIASING
    # zero units launch nothing and need no stamps
    assert probe(0, 0, 0, 0, 5, 4, 16, 0, 0, None, None, None) == MHC_SUCCESS
    assert lib.mhc_probe_wall_clock_khz(None) == MHC_ERROR_INVALID_VALUE

"""The coefficient-backward C ABI on the host (include/mhc_coeff_bwd.h):
symbols, workspace size and argument rules. No GPU: only host-only entry
points are called, and the compute entry point only with arguments it
rejects before any HIP call."""

from __future__ import annotations

import re
import subprocess

import pytest

from hyper_connection_residual_mhc_amd import _build, _lib
from hyper_connection_residual_mhc_amd._lib import (MHC_ERROR_ALIASING, MHC_ERROR_INVALID_VALUE,
                                                    MHC_SUCCESS)

GiB = 1 << 30
BASE = 16 * GiB


@pytest.fixture(scope="module")
def lib(built_library):
    return _lib.coeff_lib()


def test_header_declarations_are_all_exported(lib):
    text = re.sub(r"/\*.*?\*/", "", _build.COEFF_HEADER.read_text(), flags=re.S)
    names = sorted(set(re.findall(r"\b(mhc_\w+)\s*\(", text)))
    assert len(names) == 9, names
    out = subprocess.run(["nm", "-D", "--defined-only", str(_build.COEFF_LIB_PATH)],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (mhc_\w+)$", out, flags=re.M))
    assert set(names) <= exported, set(names) - exported
    assert set(_lib.COEFF_SIGNATURES) == set(names)
    ours = [s for s in re.findall(r"\bT (\S+)$", out, flags=re.M) if "mhc" in s or "coeff" in s]
    assert all(s.startswith("mhc_coeff_") for s in ours), ours


def test_constants_match_the_header(lib):
    text = _build.COEFF_HEADER.read_text()
    assert f"#define MHC_COEFF_ABI_VERSION {_lib.MHC_COEFF_ABI_VERSION}" in text
    assert f"#define MHC_COEFF_CHUNK {_lib.MHC_COEFF_CHUNK}" in text
    assert "#define MHC_COEFF_MAX_ROWS (1LL << 28)" in text and _lib.MHC_COEFF_MAX_ROWS == 1 << 28
    assert "#define MHC_COEFF_SCRATCH_BYTES (2LL << 20)" in text
    assert _lib.MHC_COEFF_SCRATCH_BYTES == 2 << 20
    assert lib.mhc_coeff_abi_version() == _lib.MHC_COEFF_ABI_VERSION


@pytest.mark.parametrize("n,m", [(2, 8), (4, 24), (8, 80)])
def test_workspace_bytes(lib, n, m):
    # a 256-byte header (the arrival counter), then (m + 3) sums per chunk
    f = lib.mhc_coeff_bwd_workspace_bytes
    assert f(0, n) == 0
    assert f(1, n) == 256 + (m + 3) * 4
    assert f(64, n) == 256 + (m + 3) * 4
    assert f(65, n) == 256 + 2 * (m + 3) * 4
    assert f(8192, n) == 256 + 128 * (m + 3) * 4
    assert f(1 << 28, n) == 256 + (1 << 22) * (m + 3) * 4 < (1 << 31)
    assert f(-1, n) == -1 and f((1 << 28) + 1, n) == -1


def test_launch_policy(lib):
    plan = lib.mhc_coeff_bwd_plan
    assert plan(0, 4, 0) == 2 and plan(0, 4, 1) == 2        # R = 0: the sums only
    assert plan(1, 4, 0) == 1 and plan(1, 2, 0) == 1
    assert plan(16384, 4, 0) == 1 and plan(16384, 2, 0) == 1  # up to 256 chunks: one launch
    assert plan(16385, 4, 0) == 2
    assert plan(1, 8, 0) == 2 and plan(8192, 8, 0) == 2     # n = 8: two launches
    assert plan(100, 4, 2) == 2 and plan(1 << 20, 2, 1) == 1 and plan(64, 8, 1) == 1
    assert plan(100, 4, 3) == -1 and plan(100, 4, -1) == -1 and plan(100, 5, 0) == -1


def test_workspace_bytes_rejects_bad_n(lib):
    assert lib.mhc_coeff_bwd_workspace_bytes(10, 3) == -1


class Args:
    """Disjoint fake device addresses for every tensor of an R-row call."""

    def __init__(self, lib, R, n, ws_extra=0):
        m = 2 * n + n * n
        sizes = [R * m, R * n, R * n, R * n, R * n, R * n * n, 3, R * m, m, 3]
        addr, self.p = BASE, []
        for s in sizes:
            self.p.append(addr)
            addr += ((s * 4 + 255) // 256 + 1) * 256
        self.ws = addr
        self.ws_bytes = lib.mhc_coeff_bwd_workspace_bytes(R, n) + ws_extra
        self.R, self.n, self.c = R, n, 2.0

    def tuple(self):
        p = self.p
        return (p[0], p[1], p[2], p[3], p[4], p[5], p[6], self.c, p[7], p[8], p[9], self.ws,
                self.ws_bytes, self.R, self.n)


def test_valid_arguments_pass(lib):
    for n in (2, 4, 8):
        for R in (0, 1, 65, 8192):
            assert lib.mhc_coeff_bwd_validate(*Args(lib, R, n).tuple()) == MHC_SUCCESS


def test_zero_rows_allow_null_row_tensors_but_not_sum_outputs(lib):
    a = Args(lib, 0, 4)
    t = list(a.tuple())
    for i in (0, 1, 2, 3, 4, 5, 6, 8, 11):
        t[i] = None
    assert lib.mhc_coeff_bwd_validate(*t) == MHC_SUCCESS
    t2 = list(t)
    t2[9] = None                               # grad_b
    assert lib.mhc_coeff_bwd_validate(*t2) == MHC_ERROR_INVALID_VALUE
    t2 = list(t)
    t2[10] = None                              # grad_alpha
    assert lib.mhc_coeff_bwd_validate(*t2) == MHC_ERROR_INVALID_VALUE


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4, 5, 6, 8, 9, 10, 11])
def test_null_and_misaligned_pointers(lib, idx):
    t = list(Args(lib, 100, 4).tuple())
    t0 = list(t)
    t0[idx] = None
    assert lib.mhc_coeff_bwd_validate(*t0) == MHC_ERROR_INVALID_VALUE
    t1 = list(t)
    t1[idx] = t[idx] + 2
    assert lib.mhc_coeff_bwd_validate(*t1) == MHC_ERROR_INVALID_VALUE
    assert b"aligned" in lib.mhc_coeff_last_error_message()


def test_size_and_scale_rules(lib):
    def v(**kw):
        a = Args(lib, 100, 4)
        for k, x in kw.items():
            setattr(a, k, x)
        return lib.mhc_coeff_bwd_validate(*a.tuple())
    assert v(n=3) == MHC_ERROR_INVALID_VALUE
    assert v(R=-1) == MHC_ERROR_INVALID_VALUE
    assert v(R=(1 << 28) + 1) == MHC_ERROR_INVALID_VALUE
    for c in (0.0, -0.0, -2.0, float("inf"), float("nan"), -1e-45):
        assert v(c=c) == MHC_ERROR_INVALID_VALUE, c
    # any finite positive scale, down to the smallest subnormal (post / c is
    # a division, so no reciprocal has to be representable)
    for c in (3.0, 0.5, 1e-45, 3e38):
        assert v(c=c) == MHC_SUCCESS, c
    a = Args(lib, 100, 4, ws_extra=-4)
    assert lib.mhc_coeff_bwd_validate(*a.tuple()) == MHC_ERROR_INVALID_VALUE
    assert b"workspace" in lib.mhc_coeff_last_error_message()


def test_aliasing(lib):
    a = Args(lib, 100, 4)
    t = list(a.tuple())
    t1 = list(t)
    t1[8] = t[0]                               # grad_mix on mix
    assert lib.mhc_coeff_bwd_validate(*t1) == MHC_ERROR_ALIASING
    t2 = list(t)
    t2[11] = t[8] + 64                         # workspace inside grad_mix
    assert lib.mhc_coeff_bwd_validate(*t2) == MHC_ERROR_ALIASING
    t3 = list(t)
    t3[10] = t[9] + 4                          # grad_alpha inside grad_b
    assert lib.mhc_coeff_bwd_validate(*t3) == MHC_ERROR_ALIASING
    t4 = list(t)
    t4[9] = t[6]                               # grad_b on alpha
    assert lib.mhc_coeff_bwd_validate(*t4) == MHC_ERROR_ALIASING
    assert b"overlaps" in lib.mhc_coeff_last_error_message()


def test_compute_entry_rejects_before_any_hip_call(lib):
    a = Args(lib, 100, 4)
    t = list(a.tuple())
    t[8] = t[0]
    assert lib.mhc_coeff_bwd(*t, 0, None, None, None) == MHC_ERROR_ALIASING
    t = list(a.tuple())
    t[14] = 5
    assert lib.mhc_coeff_bwd(*t, 0, None, None, None) == MHC_ERROR_INVALID_VALUE
    assert lib.mhc_coeff_bwd(*a.tuple(), 3, None, None, None) == MHC_ERROR_INVALID_VALUE
    assert b"launches" in lib.mhc_coeff_last_error_message()


def test_binding_rejects_host_tensors(lib):
    import torch
    from hyper_connection_residual_mhc_amd import coeff
    z = lambda *s: torch.zeros(s, dtype=torch.float32)
    with pytest.raises(TypeError, match="must be on a GPU"):
        coeff.mhc_coeff_bwd(z(4, 24), z(4, 4), z(4, 4), z(4, 4), z(4, 4), z(4, 16), z(3), 2.0)
    with pytest.raises(ValueError, match=r"\[R, n\]"):
        coeff.mhc_coeff_bwd(z(4, 24), z(4, 3), z(4, 4), z(4, 4), z(4, 4), z(4, 16), z(3), 2.0)


def _noalloc_max_rows(n: int) -> int:
    """Most rows the no-allocation entry point takes: whole 64-row chunks
    whose (m + 3) sums fit the scratch array after its 256-byte header."""
    m = 2 * n + n * n
    return (_lib.MHC_COEFF_SCRATCH_BYTES - 256) // ((m + 3) * 4) * 64


@pytest.mark.parametrize("n,rows", [(2, 3049984), (4, 1242560), (8, 404160)])
def test_noalloc_limit_is_the_scratch_size(lib, n, rows):
    """The header's row limits are the scratch array's capacity, and a call
    one chunk past them is refused before anything else is touched (no GPU
    needed: the size check comes first)."""
    assert _noalloc_max_rows(n) == rows
    assert lib.mhc_coeff_bwd_workspace_bytes(rows, n) <= _lib.MHC_COEFF_SCRATCH_BYTES
    assert lib.mhc_coeff_bwd_workspace_bytes(rows + 1, n) > _lib.MHC_COEFF_SCRATCH_BYTES
    m = 2 * n + n * n
    p = [BASE + k * GiB for k in range(11)]
    args = p[:7] + [2.0] + p[7:10]
    assert lib.mhc_coeff_bwd_noalloc(*args, rows + 1, n, 0, None, None,
                                     None) == MHC_ERROR_INVALID_VALUE
    assert b"scratch" in lib.mhc_coeff_last_error_message()
    assert m > 0


def test_noalloc_rejects_bad_arguments_before_any_hip_call(lib):
    p = [BASE + k * GiB for k in range(11)]
    ok_args = p[:7] + [2.0] + p[7:10]
    call = lambda args, rows=100, n=4, launches=0: lib.mhc_coeff_bwd_noalloc(
        *args, rows, n, launches, None, None, None)
    assert call(ok_args, n=3) == MHC_ERROR_INVALID_VALUE
    assert call(ok_args, rows=-1) == MHC_ERROR_INVALID_VALUE
    assert call(ok_args, launches=3) == MHC_ERROR_INVALID_VALUE
    bad_scale = p[:7] + [0.0] + p[7:10]
    assert call(bad_scale) == MHC_ERROR_INVALID_VALUE
    aliased = p[:7] + [2.0] + [p[0]] + p[8:10]          # grad_mix over mix
    assert call(aliased) == MHC_ERROR_ALIASING
    misaligned = p[:7] + [2.0] + [p[7] + 2] + p[8:10]
    assert call(misaligned) == MHC_ERROR_INVALID_VALUE


@pytest.mark.parametrize("dtype,elem", [(0, 4), (1, 2), (2, 2)])
def test_typed_argument_rules(lib, dtype, elem):
    """mhc_coeff_bwd_validate_ex: the row tensors and grad_mix need their
    element's alignment (4 bytes fp32, 2 bytes bf16 / fp16) and their sizes
    scale with it; alpha and the fp32 outputs keep 4-byte alignment; an
    unknown format is refused; the plain call is the fp32 format."""
    v = lib.mhc_coeff_bwd_validate_ex
    a = Args(lib, 100, 4)
    t = list(a.tuple())
    assert v(*t, dtype) == MHC_SUCCESS
    assert v(*t, 3) == MHC_ERROR_INVALID_VALUE and v(*t, -1) == MHC_ERROR_INVALID_VALUE
    assert b"dtype" in lib.mhc_coeff_last_error_message()
    for idx in (0, 1, 2, 3, 4, 5, 8):                       # row tensors and grad_mix
        t1 = list(t)
        t1[idx] = t[idx] + 2
        assert v(*t1, dtype) == (MHC_SUCCESS if elem == 2 else MHC_ERROR_INVALID_VALUE), idx
        t1[idx] = t[idx] + 1
        assert v(*t1, dtype) == MHC_ERROR_INVALID_VALUE, idx
    for idx in (6, 9, 10, 11):                              # alpha, grad_b, grad_alpha, workspace
        t1 = list(t)
        t1[idx] = t[idx] + 2
        assert v(*t1, dtype) == MHC_ERROR_INVALID_VALUE, idx
    # grad_mix ending right where mix starts (nothing lies below mix):
    # disjoint at the format's size; one element later it overlaps
    m, R = 24, 100
    t2 = list(t)
    t2[8] = t[0] - R * m * elem
    assert v(*t2, dtype) == MHC_SUCCESS
    t2[8] = t[0] - R * m * elem + elem
    assert v(*t2, dtype) == MHC_ERROR_ALIASING
    assert lib.mhc_coeff_bwd_validate(*t) == v(*t, 0)

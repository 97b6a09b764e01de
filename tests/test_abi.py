"""The C ABI on the host: symbols, argument rules and the launch policy.

These run without a GPU: they load the library and call only its host-only
entry points (validate / plan / status strings), which never touch a device.
Rules under test are the ones include/mhc_h_aggregate.h states.
"""

from __future__ import annotations

import ctypes
import re
import subprocess
from pathlib import Path

import pytest
import torch

from hyper_connection_residual_mhc_amd import _build, _lib, ops
from hyper_connection_residual_mhc_amd._lib import (MHC_ERROR_ALIASING, MHC_ERROR_INVALID_VALUE,
                                                    MHC_SUCCESS, MhcError)

HEADER = _build.HEADER
GiB = 1 << 30
BASE = 16 * GiB          # a 256-byte-aligned fake device address


@pytest.fixture(scope="module")
def lib(built_library):
    return _lib.lib()


def declared_functions() -> list[str]:
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mhc_\w+)\s*\(", text)))


def test_header_declarations_are_all_exported(lib, built_library):
    names = declared_functions()
    assert len(names) >= 12
    out = subprocess.run(["nm", "-D", "--defined-only", str(built_library)],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (mhc_\w+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(lib, n)
    assert set(_lib.SIGNATURES) == set(names)


def test_exports_are_c_symbols_only(built_library):
    """Nothing but the mhc_ C names is exported from the library's own code."""
    out = subprocess.run(["nm", "-D", "--defined-only", str(built_library)],
                         capture_output=True, text=True, check=True).stdout
    text_syms = re.findall(r"\bT (\S+)$", out, flags=re.M)
    ours = [s for s in text_syms if "mhc" in s or "hagg" in s]
    assert all(s.startswith("mhc_") for s in ours), ours


def test_version_and_status_strings(lib):
    assert lib.mhc_abi_version() == _lib.MHC_ABI_VERSION
    assert lib.mhc_status_string(0) == b"MHC_SUCCESS"
    assert lib.mhc_status_string(1) == b"MHC_ERROR_INVALID_VALUE"
    assert lib.mhc_status_string(2) == b"MHC_ERROR_ALIASING"
    assert lib.mhc_status_string(3) == b"MHC_ERROR_HIP"
    assert lib.mhc_status_string(99) == b"MHC_ERROR_UNKNOWN"


def fwd_ptrs(T, H, base=BASE):
    res = base
    pre = res + 8 * T * H + 4096
    out = pre + 16 * T + 4096
    return res, pre, out


def bwd_ptrs(T, H, base=BASE):
    res = base
    pre = res + 8 * T * H + 4096
    g = pre + 16 * T + 4096
    gr = g + 2 * T * H + 4096
    gp = gr + 8 * T * H + 4096
    return res, pre, g, gr, gp


def test_validate_fwd_rules(lib):
    T, H = 16, 4096
    r, p, o = fwd_ptrs(T, H)
    v = ops.mhc_h_aggregate_validate_fwd
    assert v(r, p, o, T, H) == MHC_SUCCESS
    assert v(0, 0, 0, 0, H) == MHC_SUCCESS                 # T == 0: no-op, NULL allowed
    assert v(r, p, o, -1, H) == MHC_ERROR_INVALID_VALUE
    assert v(r, p, o, T, 0) == MHC_ERROR_INVALID_VALUE
    assert v(r, p, o, 0, 0) == MHC_ERROR_INVALID_VALUE
    assert v(r, p, o, T, _lib.MHC_MAX_H + 1) == MHC_ERROR_INVALID_VALUE
    for args in ((0, p, o), (r, 0, o), (r, p, 0)):
        assert v(*args, T, H) == MHC_ERROR_INVALID_VALUE
    assert v(r + 1, p, o, T, H) == MHC_ERROR_INVALID_VALUE  # bf16 must be 2-byte aligned
    assert v(r, p + 2, o, T, H) == MHC_ERROR_INVALID_VALUE  # fp32 must be 4-byte aligned
    assert v(r, p, o + 1, T, H) == MHC_ERROR_INVALID_VALUE
    # byte counts overflowing int64
    assert v(r, p, o, (1 << 62), 8) == MHC_ERROR_INVALID_VALUE


def test_validate_fwd_aliasing(lib):
    T, H = 16, 4096
    r, p, o = fwd_ptrs(T, H)
    v = ops.mhc_h_aggregate_validate_fwd
    assert v(r, p, r, T, H) == MHC_ERROR_ALIASING                      # out == residual
    assert v(r, p, r + 8 * T * H - 2, T, H) == MHC_ERROR_ALIASING      # last element overlaps
    far = r + 64 * GiB
    assert v(r, far, r + 8 * T * H, T, H) == MHC_SUCCESS               # adjacent is fine
    assert v(r, far, far - 2 * T * H + 2, T, H) == MHC_ERROR_ALIASING  # out runs into pre
    assert v(r, far, far - 2 * T * H, T, H) == MHC_SUCCESS
    # inputs may overlap each other (both are read-only)
    assert v(r, r, o, T, H) == MHC_SUCCESS


def test_validate_bwd_rules_and_aliasing(lib):
    T, H = 8, 1279
    r, p, g, gr, gp = bwd_ptrs(T, H)
    v = ops.mhc_h_aggregate_validate_bwd
    assert v(r, p, g, gr, gp, T, H) == MHC_SUCCESS
    assert v(0, 0, 0, 0, 0, 0, H) == MHC_SUCCESS
    for i in range(5):
        args = [r, p, g, gr, gp]
        args[i] = 0
        assert v(*args, T, H) == MHC_ERROR_INVALID_VALUE, i
    assert v(r, p, g, gr, gp + 2, T, H) == MHC_ERROR_INVALID_VALUE
    assert v(r, p, g, r, gp, T, H) == MHC_ERROR_ALIASING          # grad_residual == residual
    assert v(r, p, g, gr, g, T, H) == MHC_ERROR_ALIASING          # grad_pre inside grad_out
    assert v(r, p, g, gr, gr + 64, T, H) == MHC_ERROR_ALIASING    # the two outputs overlap
    assert v(r, p, g, gr, p, T, H) == MHC_ERROR_ALIASING          # grad_pre == pre


def test_error_message_names_the_problem(lib):
    T, H = 4, 64
    r, p, o = fwd_ptrs(T, H)
    with pytest.raises(MhcError, match="ALIASING.*out overlaps input residual"):
        ops.mhc_h_aggregate_plan_fwd(r, p, r, T, H)
    with pytest.raises(MhcError, match="INVALID_VALUE.*pre is NULL"):
        ops.mhc_h_aggregate_plan_fwd(r, 0, o, T, H)


def test_forward_plan_one_wave_blocks(lib):
    """The policy uses one 64-lane wave per block at every size (the fastest
    shape measured); the grid follows T, so a 129-token batch and a 1-token
    call are different partitions of the same work."""
    r, p, o = fwd_ptrs(129, 4096)
    full, g_full = ops.mhc_h_aggregate_plan_fwd(r, p, o, 129, 4096)
    one, g_one = ops.mhc_h_aggregate_plan_fwd(r, p, o, 1, 4096)
    assert full["block_threads"] == one["block_threads"] == 64
    assert full["vec_width"] == one["vec_width"] == 8
    assert (g_full, g_one) == (129 * 8, 8)


def test_forward_plan_vector_width_follows_alignment_and_H(lib):
    T = 4
    cases = [(4096, 0, 8), (4096, 2, 1), (4096, 4, 2), (4096, 8, 4), (4100, 0, 4),
             (4098, 0, 2), (1279, 0, 1), (1, 0, 1), (8, 0, 8)]
    for H, shift, want in cases:
        r, p, o = fwd_ptrs(T, H)
        plan, _ = ops.mhc_h_aggregate_plan_fwd(r + shift, p, o, T, H)
        assert plan["vec_width"] == want, (H, shift, plan)


def test_forward_plan_grid_covers_every_unit(lib):
    for T, H in [(1, 4096), (8, 4096), (128, 7168), (1024, 7168), (8192, 7168), (3, 1279),
                 (5, 1), (2, 65536)]:
        r, p, o = fwd_ptrs(T, H)
        plan, grid = ops.mhc_h_aggregate_plan_fwd(r, p, o, T, H)
        units = H // plan["vec_width"]
        per_block = plan["block_threads"] * plan["units_per_thread"]
        assert grid == T * -(-units // per_block), (T, H, plan)
        assert grid * plan["block_threads"] >= T * units / plan["units_per_thread"]


def test_forward_overrides(lib):
    T, H = 16, 4096
    r, p, o = fwd_ptrs(T, H)
    plan, _ = ops.mhc_h_aggregate_plan_fwd(r, p, o, T, H, launch={"block_threads": 1024,
                                                                   "vec_width": 2,
                                                                   "units_per_thread": 4})
    assert plan == {"block_threads": 1024, "vec_width": 2, "units_per_thread": 4,
                    "tokens_per_block": 0, "streams_per_block": 0, "layout": 0,
                    "wave_priority": 0}
    for bad in ({"block_threads": 100}, {"block_threads": 2048}, {"vec_width": 3},
                {"units_per_thread": 3}, {"units_per_thread": 9}, {"tokens_per_block": 2},
                {"streams_per_block": 1}, {"layout": 2}, {"wave_priority": 1}):
        with pytest.raises(MhcError, match="INVALID_VALUE"):
            ops.mhc_h_aggregate_plan_fwd(r, p, o, T, H, launch=bad)
    with pytest.raises(MhcError, match="vec_width 8 not allowed"):
        ops.mhc_h_aggregate_plan_fwd(r, p, o, T, 4100, launch={"vec_width": 8})
    with pytest.raises(MhcError, match="vec_width 4 not allowed"):
        ops.mhc_h_aggregate_plan_fwd(r + 4, p, o, T, H, launch={"vec_width": 4})


def test_backward_plan_and_overrides(lib):
    T, H = 2048, 7168
    r, p, g, gr, gp = bwd_ptrs(T, H)
    SPLIT, ROWS = _lib.MHC_BWD_SPLIT, _lib.MHC_BWD_ROWS
    # long batches: one wave per (token, stream) row, a token per 256-thread block
    # (rows of at most 16 chunks of 512 elements keep 12 chunks in flight,
    # longer rows 8)
    plan, grid = ops.mhc_h_aggregate_plan_bwd(r, p, g, gr, gp, T, H)
    assert plan == {"block_threads": 256, "vec_width": 8, "units_per_thread": 12,
                    "tokens_per_block": 0, "streams_per_block": 0, "layout": ROWS,
                    "wave_priority": _lib.MHC_PRIO_FLAT}
    assert grid == T
    for H2, ring in ((8192, 12), (8200, 8)):
        plan, _ = ops.mhc_h_aggregate_plan_bwd(*bwd_ptrs(T, H2), T, H2)
        assert plan["layout"] == ROWS and plan["units_per_thread"] == ring, H2
    plan, grid = ops.mhc_h_aggregate_plan_bwd(r, p, g, gr, gp, T, H,
                                              launch={"layout": ROWS, "block_threads": 64,
                                                      "units_per_thread": 12})
    assert plan["block_threads"] == 64 and plan["units_per_thread"] == 12 and grid == 4 * T
    # the split layout, asked for or implied by its own fields
    plan, grid = ops.mhc_h_aggregate_plan_bwd(r, p, g, gr, gp, T, H, launch={"layout": SPLIT})
    assert plan == {"block_threads": 256, "vec_width": 8, "units_per_thread": 4,
                    "tokens_per_block": 1, "streams_per_block": 4, "layout": SPLIT,
                    "wave_priority": _lib.MHC_PRIO_FLAT}
    assert grid == T
    plan, grid = ops.mhc_h_aggregate_plan_bwd(r, p, g, gr, gp, T, H,
                                              launch={"tokens_per_block": 3, "vec_width": 4,
                                                      "units_per_thread": 1})
    assert plan["layout"] == SPLIT
    assert plan["tokens_per_block"] == 3 and plan["vec_width"] == 4 and grid == -(-T // 3)
    plan, grid = ops.mhc_h_aggregate_plan_bwd(r, p, g, gr, gp, T, H,
                                              launch={"streams_per_block": 2})
    assert plan["streams_per_block"] == 2 and plan["layout"] == SPLIT and grid == 2 * T
    # short batches spread each token's streams over more blocks (split layout)
    for T_, spb in ((8, 1), (127, 1), (128, 2), (135, 2)):
        plan, grid = ops.mhc_h_aggregate_plan_bwd(r, p, g, gr, gp, T_, H)
        assert plan["layout"] == SPLIT, (T_, plan)
        assert plan["streams_per_block"] == spb and grid == T_ * (4 // spb), (T_, plan)
    # from 544 rows (tokens x streams) on: the row layout
    plan, grid = ops.mhc_h_aggregate_plan_bwd(r, p, g, gr, gp, 136, H)
    assert plan["layout"] == ROWS and grid == 136
    rr, pp, gg, ggr, ggp = bwd_ptrs(1024, 2 * H)
    for n, t_split, t_rows in ((2, 271, 272), (8, 67, 68)):
        plan, _ = ops.mhc_h_aggregate_plan_bwd_n(rr, pp, gg, ggr, ggp, t_split, n, H)
        assert plan["layout"] == SPLIT, (n, plan)
        plan, _ = ops.mhc_h_aggregate_plan_bwd_n(rr, pp, gg, ggr, ggp, t_rows, n, H)
        assert plan["layout"] == ROWS, (n, plan)
    for bad in ({"block_threads": 100}, {"tokens_per_block": 5000}, {"vec_width": 16},
                {"units_per_thread": 3}, {"streams_per_block": 3}, {"layout": 3},
                {"tokens_per_block": 1, "block_threads": 128},
                {"layout": ROWS, "block_threads": 1024}, {"layout": ROWS, "units_per_thread": 2},
                {"layout": ROWS, "tokens_per_block": 1}, {"layout": ROWS, "streams_per_block": 4},
                {"layout": SPLIT, "block_threads": 64}):
        with pytest.raises(MhcError, match="INVALID_VALUE"):
            ops.mhc_h_aggregate_plan_bwd(r, p, g, gr, gp, T, H, launch=bad)
    with pytest.raises(MhcError, match="exceeds the register budget"):
        ops.mhc_h_aggregate_plan_bwd(r, p, g, gr, gp, T, H,
                                     launch={"vec_width": 1, "units_per_thread": 4,
                                             "layout": SPLIT})
    with pytest.raises(MhcError, match="exceeds the register budget"):
        ops.mhc_h_aggregate_plan_bwd(r, p, g, gr, gp, T, H,
                                     launch={"vec_width": 1, "units_per_thread": 8,
                                             "layout": ROWS})
    for bad in ({"wave_priority": 3}, {"wave_priority": -1},
                {"layout": SPLIT, "wave_priority": _lib.MHC_PRIO_PROGRESS}):
        with pytest.raises(MhcError, match="INVALID_VALUE"):
            ops.mhc_h_aggregate_plan_bwd(r, p, g, gr, gp, T, H, launch=bad)
    # grad_out misaligned by one element forces the scalar path
    plan, _ = ops.mhc_h_aggregate_plan_bwd(r, p, g + 2, gr, gp, T, H)
    assert plan["vec_width"] == 1 and plan["layout"] == ROWS and plan["units_per_thread"] == 4


def test_package_exports_every_binding_name():
    import hyper_connection_residual_mhc_amd as pkg
    from hyper_connection_residual_mhc_amd import coeff
    for name in pkg.__all__:
        got = getattr(pkg, name)
        assert got is getattr(ops, name, None) or got is getattr(coeff, name, None), name
    assert pkg.mhc_pre_h_aggregate is ops.mhc_pre_h_aggregate
    with pytest.raises(AttributeError):
        getattr(pkg, "no_such_name")


def test_binding_rejects_host_tensors_without_calling_the_library(lib):
    res = torch.zeros((2, 4, 8), dtype=torch.bfloat16)
    pre = torch.zeros((2, 4), dtype=torch.float32)
    with pytest.raises(TypeError, match="must be on a GPU"):
        ops.h_aggregate(res, pre)
    with pytest.raises(ValueError, match=r"\[T, n, H\] with n in \{2, 4, 8\}"):
        ops.h_aggregate(torch.zeros((2, 3, 8), dtype=torch.bfloat16), pre)
    with pytest.raises(ValueError, match=r"\[T, 4, H\]"):
        ops.mhc_h_aggregate_fwd(torch.zeros((2, 2, 8), dtype=torch.bfloat16), pre, res)


def test_compute_call_with_invalid_args_returns_before_any_hip_call(lib):
    """Argument errors are reported by the compute entry points themselves
    (no launch is attempted, so this runs without a GPU)."""
    T, H = 4, 64
    r, p, o = fwd_ptrs(T, H)
    assert lib.mhc_h_aggregate_fwd(r, p, r, T, H, None) == MHC_ERROR_ALIASING
    assert lib.mhc_h_aggregate_fwd(r, p, o, -3, H, None) == MHC_ERROR_INVALID_VALUE
    assert lib.mhc_h_aggregate_fwd(0, 0, 0, 0, H, None) == MHC_SUCCESS
    rr, pp, g, gr, gp = bwd_ptrs(T, H)
    assert lib.mhc_h_aggregate_bwd(rr, pp, g, gr, gr, T, H, None) == MHC_ERROR_ALIASING
    bad = _lib.mhc_launch(block_threads=64)
    assert lib.mhc_h_aggregate_bwd_ex(rr, pp, g, gr, gp, T, H, None,
                                      ctypes.byref(bad)) == MHC_ERROR_INVALID_VALUE
    assert lib.mhc_h_aggregate_fwd_timed(r, p, r, T, H, None, None, None,
                                         None) == MHC_ERROR_ALIASING
    assert lib.mhc_h_aggregate_bwd_timed(rr, pp, g, gr, gp, -1, H, None, None, None,
                                         None) == MHC_ERROR_INVALID_VALUE


def test_missing_library_raises_import_error(tmp_path):
    with pytest.raises(ImportError, match="missing"):
        _lib.open_checked(Path(tmp_path) / "absent.so", _build.SRC, _lib.SIGNATURES,
                          "mhc_abi_version", _lib.MHC_ABI_VERSION)


def test_stale_library_is_refused(built_library, tmp_path):
    """A library whose recorded digest does not match the sources in the tree
    (or that has no record) is not loaded; the same file with a matching
    record is."""
    copy = Path(tmp_path) / built_library.name
    copy.write_bytes(built_library.read_bytes())
    info = _build.build_info_path(copy)
    args = (copy, _build.SRC, _lib.SIGNATURES, "mhc_abi_version", _lib.MHC_ABI_VERSION)
    with pytest.raises(ImportError, match="other sources"):
        _lib.open_checked(*args)                                    # no record
    info.write_text('{"source_digest": "' + "0" * 64 + '"}')
    with pytest.raises(ImportError, match="other sources"):
        _lib.open_checked(*args)                                    # stale record
    info.write_text('{"source_digest": "' + _build.source_digest(_build.SRC) + '"}')
    assert _lib.open_checked(*args).mhc_abi_version() == _lib.MHC_ABI_VERSION


def test_source_digest_follows_sources_headers_and_flags(monkeypatch, tmp_path):
    """The digest changes with the source, any header and the flags, and
    does not depend on where the repository sits."""
    base = _build.source_digest(_build.SRC)
    assert base == _build.source_digest(_build.SRC)
    assert base != _build.source_digest(_build.COEFF_SRC)
    assert base != _build.source_digest(_build.SRC, ["-DX=1"])
    monkeypatch.setitem(_build.SOURCE_FLAGS, _build.SRC, [])
    assert base != _build.source_digest(_build.SRC)
    monkeypatch.undo()
    src = Path(tmp_path) / _build.SRC.name
    src.write_bytes(_build.SRC.read_bytes() + b"\n")
    assert base != _build.source_digest(src)
    assert all(str(_build.REPO_DIR) not in f or f == str(_build.INCLUDE_DIR)
               for f in _build.COMMON_FLAGS)


def test_built_libraries_match_the_tree(built_library):
    """The libraries in the tree were built from the current sources."""
    assert _build.library_is_built()


def test_accumulating_backward_plan(lib):
    """The accumulating backward also loads the stored gradient, so its ring
    is smaller where the register budget requires it; it follows the same
    layout and streams-per-block policy and the same argument rules."""
    T, H = 2048, 7168
    r, p, g, gr, gp = bwd_ptrs(T, H)
    SPLIT, ROWS = _lib.MHC_BWD_SPLIT, _lib.MHC_BWD_ROWS
    plan, grid = ops.mhc_h_aggregate_plan_bwd_acc(r, p, g, gr, gp, T, H)
    assert plan["layout"] == ROWS and plan["units_per_thread"] == 8 and grid == T
    plan, grid = ops.mhc_h_aggregate_plan_bwd_acc(r, p, g, gr, gp, T, H, launch={"layout": SPLIT})
    assert plan["streams_per_block"] == 4 and plan["units_per_thread"] == 2 and grid == T
    plan, _ = ops.mhc_h_aggregate_plan_bwd_acc(r, p, g, gr, gp, 64, H)
    assert plan["layout"] == SPLIT
    assert plan["streams_per_block"] == 1 and plan["units_per_thread"] == 4
    with pytest.raises(MhcError, match="exceeds the register budget"):
        ops.mhc_h_aggregate_plan_bwd_acc(r, p, g, gr, gp, T, H,
                                         launch={"units_per_thread": 4, "layout": SPLIT})
    with pytest.raises(MhcError, match="exceeds the register budget"):
        ops.mhc_h_aggregate_plan_bwd_acc(r, p, g, gr, gp, T, H,
                                         launch={"units_per_thread": 12, "layout": ROWS})
    # scalar accesses: the row layout does not fit the budget, the policy splits
    plan, _ = ops.mhc_h_aggregate_plan_bwd_acc(r, p, g + 2, gr, gp, T, H)
    assert plan["vec_width"] == 1 and plan["layout"] == SPLIT
    with pytest.raises(MhcError, match="row layout exceeds the register budget"):
        ops.mhc_h_aggregate_plan_bwd_acc(r, p, g + 2, gr, gp, T, H, launch={"layout": ROWS})
    with pytest.raises(MhcError, match="ALIASING"):
        ops.mhc_h_aggregate_plan_bwd_acc(r, p, g, r, gp, T, H)
    assert lib.mhc_h_aggregate_bwd_acc(r, p, g, gr, gr, T, H, None, None, None,
                                       None) == MHC_ERROR_ALIASING
    assert lib.mhc_h_aggregate_bwd_acc(0, 0, 0, 0, 0, 0, H, None, None, None,
                                       None) == MHC_SUCCESS


def test_expansion_rate_rules(lib):
    """n must be 2, 4 or 8; sizes scale with n; streams_per_block <= n; the
    register budget caps the forward batch at n = 8."""
    T, H = 64, 4096
    r, p, o = fwd_ptrs(T, H * 2)   # room for n = 8
    for n in (2, 4, 8):
        plan, grid = ops.mhc_h_aggregate_plan_fwd_n(r, p, o, T, n, H)
        assert plan["vec_width"] == 8 and grid == T * (H // 8 // 64)
    for bad_n in (0, 1, 3, 16):
        with pytest.raises(MhcError, match="expansion rate n must be 2, 4 or 8"):
            ops.mhc_h_aggregate_plan_fwd_n(r, p, o, T, bad_n, H)
    with pytest.raises(MhcError, match="exceeds the register budget"):
        ops.mhc_h_aggregate_plan_fwd_n(r, p, o, T, 8, H, launch={"units_per_thread": 4})
    # n = 8 residual is twice the n = 4 one: out right after 4-stream bytes overlaps
    with pytest.raises(MhcError, match="ALIASING"):
        ops.mhc_h_aggregate_plan_fwd_n(r, r + 8 * T * H * 2, r + 8 * T * H, T, 8, H)
    rr, pp, g, gr, gp = bwd_ptrs(1024, H * 2)
    # row layout: four rows per block (two tokens at n = 2, half a token at 8)
    plan, grid = ops.mhc_h_aggregate_plan_bwd_n(rr, pp, g, gr, gp, 1024, 2, H)
    assert plan["block_threads"] == 256 and grid == 512
    plan, grid = ops.mhc_h_aggregate_plan_bwd_n(rr, pp, g, gr, gp, 1024, 8, H)
    assert plan["block_threads"] == 256 and grid == 2048
    plan, grid = ops.mhc_h_aggregate_plan_bwd_n(rr, pp, g, gr, gp, 1024, 2, H,
                                                launch={"layout": _lib.MHC_BWD_SPLIT})
    assert plan["streams_per_block"] == 2 and grid == 1024
    plan, grid = ops.mhc_h_aggregate_plan_bwd_n(rr, pp, g, gr, gp, 1024, 8, H,
                                                launch={"layout": _lib.MHC_BWD_SPLIT})
    assert plan["streams_per_block"] == 4 and grid == 2048
    with pytest.raises(MhcError, match="exceeds the 2 streams"):
        ops.mhc_h_aggregate_plan_bwd_n(rr, pp, g, gr, gp, 8, 2, H,
                                       launch={"streams_per_block": 4})
    assert lib.mhc_h_aggregate_bwd_n(rr, pp, g, gr, gp, 8, 4, H, 2, None, None, None,
                                     None) == MHC_ERROR_INVALID_VALUE


def test_backward_issue_priority_policy(lib):
    """Progress priority for the written backward exactly when every row of
    the call has a wave slot from the start: T * n <= 16 x compute units
    (256 here: the plan is computed without a device, or on an MI355X),
    rows of at most 16 chunks of 16-byte accesses; overridable both ways
    within those rows, also for the accumulating backward."""
    FLAT, PROGRESS = _lib.MHC_PRIO_FLAT, _lib.MHC_PRIO_PROGRESS
    H = 7168
    r, p, g, gr, gp = bwd_ptrs(2048, 2 * H)
    prio = lambda T, n=4, H=H, acc=0, **launch: ops.mhc_h_aggregate_plan_bwd_n(
        r, p, g, gr, gp, T, n, H, accumulate=acc, launch=launch or None)[0]["wave_priority"]
    assert prio(1024) == PROGRESS and prio(1025) == FLAT and prio(136) == PROGRESS
    assert prio(1024, acc=1) == FLAT and prio(1024, acc=1, wave_priority=PROGRESS) == PROGRESS
    assert prio(2048, n=2) == PROGRESS and prio(2049, n=2) == FLAT
    assert prio(512, n=8) == PROGRESS and prio(513, n=8) == FLAT
    assert prio(1024, H=8192) == PROGRESS and prio(1024, H=8200) == FLAT   # looping rows
    assert prio(100) == FLAT                                                 # split layout
    assert prio(2048, wave_priority=PROGRESS) == PROGRESS
    assert prio(1024, wave_priority=FLAT) == FLAT
    assert prio(100, wave_priority=FLAT) == FLAT
    for T, H2, launch in ((1024, 8200, {}), (1024, H, {"vec_width": 4}),
                          (100, H, {"layout": _lib.MHC_BWD_SPLIT})):
        with pytest.raises(MhcError, match="INVALID_VALUE"):
            ops.mhc_h_aggregate_plan_bwd_n(r, p, g, gr, gp, T, 4, H2,
                                           launch=dict(launch, wave_priority=PROGRESS))

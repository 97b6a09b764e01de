"""Build-time guards of the arithmetic contract, checked on this library's
own gfx950 machine code (compiled here; no GPU needed).

* no fused or packed fp32 arithmetic: the page's kernel computes every fp32
  product and sum as a separate round-to-nearest operation (section Batch
  invariance of "Add batch-invariant h_aggregate kernel");
* fp32 denormals kept (no flush-to-zero) in every kernel descriptor;
* bf16 results produced by the round-to-nearest-even pack conversion;
* a fast-math build is refused at compile time;
* no register spills to scratch in the kernels;
* no store of more than 8 bytes is followed at once by an instruction that
  overwrites its data registers (gfx950 reads such data over several cycles;
  an immediate overwrite was measured to corrupt the last lanes' data);
* no scalar memory writes;
* no division in the h_aggregate kernels; in the coefficient kernels the one
  fp32 division of the post gate (post / c) is the compiler's correctly
  rounded expansion, and the fused multiply-adds of that expansion are the
  only fused operations in them;
* no __builtin_bit_cast of a vector element in the kernel sources (this
  toolchain turned `__builtin_bit_cast(float, v[e])` on a 4-wide vector into
  a copy of element 0 and shrank the vector load to one dword; the
  kernels copy an element into a scalar first);
* the product path never imports the oracle.

All three library sources are checked (the h_aggregate kernels, the
coefficient-backward epilogue's kernels and the measurement library's
probes).
"""

from __future__ import annotations

import re
import subprocess
from pathlib import Path

import pytest

from hyper_connection_residual_mhc_amd import _build

# Fused or packed fp32 instructions, in any encoding (_e32, _e64, _dpp, _sdwa).
FORBIDDEN = re.compile(
    r"\b(v_fma_f32|v_fmac_f32|v_mad_f32|v_mac_f32|v_fma_legacy_f32|v_fmac_legacy_f32|"
    r"v_mad_legacy_f32|v_fma_mix\w*|v_mad_mix\w*|v_dot2\w*|v_pk_fma_f32|v_pk_mul_f32|"
    r"v_pk_add_f32|v_fma_f64|v_fma_f16|v_pk_fma_f16)(_e32|_e64|_dpp|_sdwa)?\b")


SOURCES = [_build.SRC, _build.COEFF_SRC, _build.PROBE_SRC]


@pytest.fixture(scope="module", params=SOURCES, ids=lambda p: p.stem)
def asm(request, tmp_path_factory) -> str:
    out = tmp_path_factory.mktemp("asm") / f"{request.param.stem}.s"
    return _build.device_asm(out, src=request.param).read_text()


def kernel_blocks(asm: str) -> dict[str, str]:
    """Instruction text of each kernel, keyed by symbol."""
    blocks = {}
    for m in re.finditer(r"^(_Z\w+):[^\n]*$(.*?)^\.Lfunc_end\d+:", asm, flags=re.M | re.S):
        blocks[m.group(1)] = m.group(2)
    return blocks


def test_kernels_present(asm):
    names = list(kernel_blocks(asm))
    if any("coeff_" in n for n in names):
        # 3 rates x (fp32 + bf16 and fp16 with 16- or 32-bit accesses)
        assert sum("coeff_partial_kernel" in n for n in names) == 15
        assert sum("coeff_reduce_kernel" in n for n in names) == 1
        assert sum("coeff_clear_counter_kernel" in n for n in names) == 1
        assert not any("hagg_" in n or "probe" in n for n in names)
        return
    if any("probe" in n for n in names):
        assert sum("bf16_probe_kernel" in n for n in names) == 1
        assert sum("stream_probe_kernel" in n for n in names) == 6
        assert sum("clock_probe_kernel" in n for n in names) == 6
        assert not any("hagg_" in n or "coeff_" in n for n in names)
        return
    assert any("hagg_fwd_kernel" in n for n in names)
    assert any("hagg_bwd_kernel" in n for n in names)
    assert any("hagg_bwd_rows_kernel" in n for n in names)
    assert not any("probe" in n or "coeff_" in n for n in names)


def test_no_scalar_memory_writes(asm):
    """Every store goes through the vector memory path."""
    hits = re.findall(r"^\s*(s_store\w*|s_buffer_store\w*|s_scratch_store\w*|s_atomic\w*|"
                      r"s_buffer_atomic\w*|s_dcache_wb\w*|s_dcache_discard\w*)", asm, flags=re.M)
    assert not hits, sorted(set(hits))


DIVISION_FMA = re.compile(r"^\s*(v_fma_f32|v_fmac_f32\w*)\b")


def division_spans(ins: list[str]) -> list[tuple[int, int]]:
    """[first, last] instruction indices of each run of fp32 divisions: from
    a v_div_scale_f32 that starts one to the v_div_fixup_f32 that completes
    the last division begun in the run (each division has two div_scale and
    one div_fixup; the compiler may interleave several)."""
    spans, start, scales, fixups = [], None, 0, 0
    for i, line in enumerate(ins):
        op = line.split()[0] if line.split() else ""
        if op == "v_div_scale_f32":
            if start is None:
                start, scales, fixups = i, 0, 0
            scales += 1
        elif op == "v_div_fixup_f32" and start is not None:
            fixups += 1
            if 2 * fixups == scales:
                spans.append((start, i))
                start = None
    assert start is None, "unterminated division"
    return spans


def fused_outside_divisions(body: str) -> list[str]:
    """Forbidden instructions of a kernel, except the fused multiply-adds of
    the division expansion (five per division, inside its span)."""
    ins = instructions(body)
    spans = division_spans(ins)
    inside = set()
    for a, b in spans:
        fmas = [i for i in range(a, b + 1) if DIVISION_FMA.match(ins[i])]
        divs = sum(1 for i in range(a, b + 1) if ins[i].split()[0] == "v_div_fixup_f32")
        assert len(fmas) == 5 * divs, (a, b, len(fmas), divs)
        inside.update(fmas)
    return [ins[i].strip() for i in range(len(ins))
            if i not in inside and FORBIDDEN.search(ins[i])]


def test_no_fused_or_packed_float_ops(asm):
    for name, body in kernel_blocks(asm).items():
        if "coeff_" in name:
            hits = fused_outside_divisions(body)
        else:
            hits = [m.group(0) for m in FORBIDDEN.finditer(body)]
        assert not hits, f"{name}: {sorted(set(hits))}"


def test_forbidden_pattern_covers_every_encoding():
    for text in ("v_fma_f32 v1, v2, v3, v4", "v_fmac_f32_e32 v2, v4, v2",
                 "v_fmac_f32_e64 v2, v4, v2", "v_mac_f32_e32 v1, v2, v3",
                 "v_pk_mul_f32 v[0:1], v[2:3], v[4:5]", "v_dot2_f32_bf16 v1, v2, v3, v4",
                 "v_fma_mix_f32 v1, v2, v3, v4"):
        assert FORBIDDEN.search(text), text
    for text in ("v_mul_f32_e32 v1, v2, v3", "v_add_f32_e32 v1, v2, v3",
                 "v_cvt_pk_bf16_f32 v1, v2, v3", "v_div_fmas_f32 v1, v2, v3, v4"):
        assert not FORBIDDEN.search(text), text


def test_division_scan_allows_only_the_expansion():
    """The scan accepts a division's own fused steps and flags any other."""
    div = ["v_div_scale_f32 v1, s[2:3], s10, s10, v0", "v_rcp_f32_e32 v2, v1",
           "v_div_scale_f32 v3, vcc, v0, s10, v0", "v_fma_f32 v4, -v1, v2, 1.0",
           "v_fmac_f32_e32 v2, v4, v2", "v_mul_f32_e32 v4, v3, v2",
           "v_fma_f32 v5, -v1, v4, v3", "v_fmac_f32_e32 v4, v5, v2",
           "v_fma_f32 v1, -v1, v4, v3", "v_div_fmas_f32 v1, v1, v2, v4",
           "v_div_fixup_f32 v1, v1, s10, v0"]
    body = "\n".join("\t" + x for x in div)
    assert fused_outside_divisions(body) == []
    assert fused_outside_divisions(body + "\n\tv_fma_f32 v7, v1, v2, v3") == ["v_fma_f32 v7, v1, v2, v3"]
    assert fused_outside_divisions("\tv_fmac_f32_e32 v2, v4, v2") == ["v_fmac_f32_e32 v2, v4, v2"]
    with pytest.raises(AssertionError):
        fused_outside_divisions("\n".join("\t" + x for x in div[:4] + div[9:]))


def test_separate_fp32_mul_and_add_present(asm):
    for name, body in kernel_blocks(asm).items():
        if "hagg_" in name or "coeff_partial" in name:
            assert "v_mul_f32" in body and "v_add_f32" in body, name


def test_bf16_results_use_rne_pack_conversion(asm):
    for name, body in kernel_blocks(asm).items():
        if "stream_probe_kernel" in name or "clock_probe_kernel" in name or "coeff_" in name:
            continue  # no bf16 value produced (byte streams; fp32 in and out)
        assert "v_cvt_pk_bf16_f32" in body, name


def test_divisions_only_where_the_operation_has_one(asm):
    """The h_aggregate kernels divide nothing; the coefficient chunk stage
    divides once per post column (post / c), the reduction never."""
    for name, body in kernel_blocks(asm).items():
        fixups = len(re.findall(r"^\s*v_div_fixup_f32\b", body, flags=re.M))
        if "hagg_" in name:
            assert not re.search(r"\bv_(div_\w+|rcp_\w+)", body), name
        elif "coeff_reduce" in name or "coeff_clear" in name:
            assert fixups == 0, name
        elif "coeff_" in name:
            n = int(re.search(r"kernelILi(\d+)E", name).group(1))
            assert fixups == n, (name, fixups)


STORE_WIDE = re.compile(
    r"^\s*(buffer_store_dwordx[34]|global_store_dwordx[34]|flat_store_dwordx[34]|"
    r"scratch_store_dwordx[34])\s+(.*)$")


def _regs(text: str) -> set[int]:
    """VGPR numbers named by one operand (v7 or v[4:7])."""
    m = re.fullmatch(r"v(\d+)", text)
    if m:
        return {int(m.group(1))}
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", text)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


def store_data_regs(line: str) -> set[int]:
    """Data VGPRs of a wide store (buffer: first operand; global/flat:
    second operand)."""
    m = STORE_WIDE.match(line)
    ops = [o.strip() for o in m.group(2).split(",")]
    return _regs(ops[0] if m.group(1).startswith("buffer") else ops[1])


def written_vgprs(line: str) -> set[int]:
    """VGPRs written by a VALU instruction (its first operand)."""
    t = line.strip()
    if not t.startswith("v_"):
        return set()
    parts = t.split(None, 1)
    if len(parts) < 2:
        return set()
    return _regs(parts[1].split(",")[0].strip())


def instructions(body: str) -> list[str]:
    out = []
    for ln in body.splitlines():
        t = ln.split(";")[0].rstrip()
        if not t.strip() or t.strip().startswith(".") or t.rstrip().endswith(":"):
            continue
        out.append(t)
    return out


def test_no_immediate_overwrite_of_wide_store_data(asm):
    checked = 0
    for name, body in kernel_blocks(asm).items():
        ins = instructions(body)
        for i, line in enumerate(ins[:-1]):
            if not STORE_WIDE.match(line):
                continue
            checked += 1
            clash = store_data_regs(line) & written_vgprs(ins[i + 1])
            assert not clash, f"{name}: '{line.strip()}' then '{ins[i + 1].strip()}'"
    assert checked > 0


def test_hazard_scan_detects_the_pattern():
    """The scan itself flags the measured corrupting sequence."""
    body = ("\tbuffer_store_dwordx4 v[60:63], v56, s[36:39], s22 offen nt\n"
            "\tv_lshlrev_b32_e32 v61, 16, v30\n")
    ins = instructions(body)
    assert store_data_regs(ins[0]) & written_vgprs(ins[1]) == {61}
    ok = ("\tbuffer_store_dwordx4 v[60:63], v56, s[36:39], 0 offen nt\n"
          "\ts_nop 0\n\tv_lshlrev_b32_e32 v61, 16, v30\n")
    ins = instructions(ok)
    assert not store_data_regs(ins[0]) & written_vgprs(ins[1])


def test_fp32_denormals_kept_in_every_kernel(asm):
    modes = re.findall(r"\.amdhsa_float_denorm_mode_32\s+(\d+)", asm)
    assert modes and all(m == "3" for m in modes), modes


def test_no_scratch_spills(asm):
    spills = re.findall(r"\.vgpr_spill_count:\s+(\d+)", asm)
    assert spills and all(s == "0" for s in spills), spills
    assert "scratch_store" not in asm and "buffer_store_dword off" not in asm


@pytest.mark.parametrize("src", SOURCES, ids=lambda p: p.stem)
def test_fast_math_build_is_refused(tmp_path, src):
    cmd = [_build.hipcc(), *_build.COMMON_FLAGS, "-ffast-math", "--cuda-device-only", "-S",
           str(src), "-o", str(tmp_path / "fm.s")]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    assert proc.returncode != 0
    assert "must not be built with fast-math" in proc.stdout + proc.stderr


def test_build_flags_fix_the_contract():
    flags = " ".join(_build.COMMON_FLAGS)
    assert "--offload-arch=gfx950" in flags
    assert "-ffp-contract=off" in flags
    assert "-packed-fp32-ops" in flags
    assert "fast-math" not in flags and "-ffast" not in flags
    for path in SOURCES:
        assert "#pragma clang fp contract(off)" in path.read_text(), path


def test_product_path_does_not_touch_the_oracle():
    pkg = Path(_build.PKG_DIR)
    for f in list(pkg.rglob("*.py")) + list(pkg.rglob("*.hip")) + list(pkg.rglob("*.h")):
        text = f.read_text()
        assert not re.search(r"^\s*(from|import)\s+oracle\b", text, flags=re.M), f
        assert "oracle/" not in text, f


BIT_CAST_OF_ELEMENT = re.compile(r"__builtin_bit_cast\(\s*[\w:]+\s*,\s*[\w.]+\s*\[")


def test_no_bit_cast_of_a_vector_element():
    csrc = Path(_build.PKG_DIR) / "csrc"
    for f in sorted(list(csrc.glob("*.hip")) + list(csrc.glob("*.h"))):
        hits = [line for line in f.read_text().splitlines() if BIT_CAST_OF_ELEMENT.search(line)]
        assert not hits, (f.name, hits)


def test_bit_cast_scan_detects_the_pattern():
    assert BIT_CAST_OF_ELEMENT.search("dst[e] = __builtin_bit_cast(float, v[e]);")
    assert BIT_CAST_OF_ELEMENT.search("x = __builtin_bit_cast(float, a.b[1]);")
    assert not BIT_CAST_OF_ELEMENT.search("x = __builtin_bit_cast(float, u);")
    assert not BIT_CAST_OF_ELEMENT.search(
        "return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, o, 0, 0));")

"""Build-time guards of the arithmetic contract, checked on this library's
own gfx950 machine code (compiled here; no GPU needed).

* no fused or packed fp32 arithmetic: the page's kernel computes every fp32
  product and sum as a separate round-to-nearest operation (section Batch
  invariance of "Add batch-invariant h_aggregate kernel");
* fp32 denormals kept (no flush-to-zero) in every kernel descriptor;
* bf16 results produced by the round-to-nearest-even pack conversion;
* a fast-math build is refused at compile time;
* no register spills to scratch in the kernels;
* the product path never imports the oracle.
"""

from __future__ import annotations

import re
import subprocess
from pathlib import Path

import pytest

from hyper_connection_residual_mhc_amd import _build

FORBIDDEN = re.compile(
    r"\b(v_fma_f32|v_fmac_f32|v_mad_f32|v_mac_f32|v_fma_legacy_f32|v_fmac_legacy_f32|"
    r"v_mad_legacy_f32|v_fma_mix\w*|v_mad_mix\w*|v_dot2\w*|v_pk_fma_f32|v_pk_mul_f32|"
    r"v_pk_add_f32|v_fma_f64|v_fma_f16|v_pk_fma_f16)\b")


@pytest.fixture(scope="module")
def asm(tmp_path_factory) -> str:
    out = tmp_path_factory.mktemp("asm") / "mhc.s"
    return _build.device_asm(out).read_text()


def kernel_blocks(asm: str) -> dict[str, str]:
    """Instruction text of each kernel, keyed by symbol."""
    blocks = {}
    for m in re.finditer(r"^(_Z\w+):[^\n]*$(.*?)^\.Lfunc_end\d+:", asm, flags=re.M | re.S):
        blocks[m.group(1)] = m.group(2)
    return blocks


def test_kernels_present(asm):
    names = list(kernel_blocks(asm))
    assert any("hagg_fwd_kernel" in n for n in names)
    assert any("hagg_bwd_kernel" in n for n in names)
    assert any("bf16_probe_kernel" in n for n in names)


def test_no_fused_or_packed_float_ops(asm):
    for name, body in kernel_blocks(asm).items():
        hits = FORBIDDEN.findall(body)
        assert not hits, f"{name}: {sorted(set(hits))}"


def test_separate_fp32_mul_and_add_present(asm):
    for name, body in kernel_blocks(asm).items():
        if "hagg_" in name:
            assert "v_mul_f32" in body and "v_add_f32" in body, name


def test_bf16_results_use_rne_pack_conversion(asm):
    for name, body in kernel_blocks(asm).items():
        assert "v_cvt_pk_bf16_f32" in body, name


def test_fp32_denormals_kept_in_every_kernel(asm):
    modes = re.findall(r"\.amdhsa_float_denorm_mode_32\s+(\d+)", asm)
    assert modes and all(m == "3" for m in modes), modes


def test_no_scratch_spills(asm):
    spills = re.findall(r"\.vgpr_spill_count:\s+(\d+)", asm)
    assert spills and all(s == "0" for s in spills), spills
    assert "scratch_store" not in asm and "buffer_store_dword off" not in asm


def test_fast_math_build_is_refused(tmp_path):
    cmd = [_build.hipcc(), *_build.COMMON_FLAGS, "-ffast-math", "--cuda-device-only", "-S",
           str(_build.SRC), "-o", str(tmp_path / "fm.s")]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    assert proc.returncode != 0
    assert "must not be built with fast-math" in proc.stdout + proc.stderr


def test_build_flags_fix_the_contract():
    flags = " ".join(_build.COMMON_FLAGS)
    assert "--offload-arch=gfx950" in flags
    assert "-ffp-contract=off" in flags
    assert "-packed-fp32-ops" in flags
    assert "fast-math" not in flags and "-ffast" not in flags
    src = _build.SRC.read_text()
    assert "#pragma clang fp contract(off)" in src


def test_product_path_does_not_touch_the_oracle():
    pkg = Path(_build.PKG_DIR)
    for f in list(pkg.rglob("*.py")) + list(pkg.rglob("*.hip")) + list(pkg.rglob("*.h")):
        text = f.read_text()
        assert not re.search(r"^\s*(from|import)\s+oracle\b", text, flags=re.M), f
        assert "oracle/" not in text, f

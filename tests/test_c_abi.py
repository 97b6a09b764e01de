"""The boundary from plain C: tests/c_abi/host_calls.c includes both public
headers as C99 with warnings as errors, links against both built libraries
and exercises the host-only entry points (no GPU needed)."""

from __future__ import annotations

import shutil
import subprocess

import pytest

from hyper_connection_residual_mhc_amd import _build

SRC = _build.REPO_DIR / "tests" / "c_abi" / "host_calls.c"


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_caller_compiles_links_and_passes(built_library, tmp_path):
    exe = tmp_path / "host_calls"
    lib_dir = built_library.parent
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", str(_build.INCLUDE_DIR), str(SRC), "-o", str(exe),
                    "-L", str(lib_dir), "-lmhc_h_aggregate", "-lmhc_coeff_bwd",
                    f"-Wl,-rpath,{lib_dir}"],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert "c abi ok" in r.stdout

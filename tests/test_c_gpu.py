"""Both operation libraries on the GPU from a plain C99 program
(tests/c_abi/gpu_calls.c), including the coefficient epilogue's bf16 and
no-allocation entry points:
device memory from the HIP runtime, the null stream, no Python or torch in
the process. Its outputs are compared with the oracle byte for byte."""

from __future__ import annotations

import shutil
import subprocess

import numpy as np
import pytest

from conftest import assert_bytes_equal
from gpu_util import say
from hyper_connection_residual_mhc_amd import _build
from hyper_connection_residual_mhc_amd.workloads import make_coeff_inputs, make_inputs
from oracle import coeff_bwd as CB
from oracle import h_aggregate as O

pytestmark = pytest.mark.gpu

SRC = _build.REPO_DIR / "tests" / "c_abi" / "gpu_calls.c"
ROCM = "/opt/rocm"


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_program_on_the_gpu_matches_the_oracle(built_library, tmp_path):
    exe = tmp_path / "gpu_calls"
    lib_dir = _build.LIB_DIR
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", str(_build.INCLUDE_DIR), "-isystem", f"{ROCM}/include", str(SRC),
                    "-o", str(exe), "-L", str(lib_dir), "-lmhc_h_aggregate", "-lmhc_coeff_bwd",
                    f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{lib_dir}",
                    f"-Wl,-rpath,{ROCM}/lib"], check=True, capture_output=True, text=True)
    T, H, R = 129, 4100, 300
    host = make_inputs(T, H, seed=70, grad=True)
    for k in ("residual", "pre", "grad_out"):
        np.ascontiguousarray(host[k]).tofile(tmp_path / f"{k}.bin")
    ch = make_coeff_inputs(R, 4, seed=71)
    for k in ("mix", "pre", "post", "grad_pre", "grad_post", "grad_res", "alpha"):
        np.ascontiguousarray(ch[k]).tofile(tmp_path / f"c_{k}.bin")
    c16 = {k: CB.narrow(ch[k], "bf16") for k in CB.ROW_INPUTS}
    for k, v in c16.items():
        np.ascontiguousarray(v).tofile(tmp_path / f"c16_{k}.bin")
    say(f"C program on the GPU: T={T} H={H} R={R}")
    r = subprocess.run([str(exe), str(tmp_path), str(T), str(H), str(R)], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c gpu calls ok" in r.stdout

    read = lambda name, dt, shape: np.fromfile(tmp_path / name, dtype=dt).reshape(shape)
    assert_bytes_equal(read("out.bin", np.uint16, (T, H)),
                       O.h_aggregate_fwd(host["residual"], host["pre"]), "C forward")
    want_gr, want_gp = O.h_aggregate_bwd(host["residual"], host["pre"], host["grad_out"])
    assert_bytes_equal(read("grad_residual.bin", np.uint16, (T, 4, H)), want_gr, "C grad_residual")
    assert_bytes_equal(read("grad_pre.bin", np.float32, (T, 4)), want_gp, "C grad_pre")
    want = CB.coeff_bwd(*(ch[k] for k in ("mix", "pre", "post", "grad_pre", "grad_post",
                                          "grad_res", "alpha")), 2.0, 4)
    assert_bytes_equal(read("c_grad_mix.bin", np.float32, (R, 24)), want[0], "C grad_mix")
    assert_bytes_equal(read("c_grad_b.bin", np.float32, (24,)), want[1], "C grad_b")
    assert_bytes_equal(read("c_grad_alpha.bin", np.float32, (3,)), want[2], "C grad_alpha")
    assert_bytes_equal(read("c_na_grad_mix.bin", np.float32, (R, 24)), want[0], "C noalloc grad_mix")
    assert_bytes_equal(read("c_na_grad_b.bin", np.float32, (24,)), want[1], "C noalloc grad_b")
    assert_bytes_equal(read("c_na_grad_alpha.bin", np.float32, (3,)), want[2],
                       "C noalloc grad_alpha")
    w16 = CB.coeff_bwd_typed(*(c16[k] for k in CB.ROW_INPUTS), ch["alpha"], 2.0, 4, "bf16")
    assert_bytes_equal(read("c16_grad_mix.bin", np.uint16, (R, 24)), w16[0], "C bf16 grad_mix")
    assert_bytes_equal(read("c16_grad_b.bin", np.float32, (24,)), w16[1], "C bf16 grad_b")
    assert_bytes_equal(read("c16_grad_alpha.bin", np.float32, (3,)), w16[2], "C bf16 grad_alpha")

"""Planted mistakes in the oracles must fail their pins.

Each mutant changes one plausible thing in a copy of an oracle module: an
extra or missing rounding, a fused operation, a transposed or dropped
operand, a wrong index, association, order or constant. The module's pin
file (tests/test_oracle.py or tests/test_coeff_oracle.py) then runs against
the copy in a subprocess and must report failing tests. A control run of the
unchanged copies must pass, so that a failure means the pins caught the
mutant and not that the harness is broken. The repository's own files are
never modified. CPU only.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

import pytest

REPO = Path(__file__).resolve().parent.parent
PKG = "hyper_connection_residual_mhc_amd"

PINS = {
    "h_aggregate": ["tests/test_oracle.py", "--deselect",
                    "tests/test_oracle.py::"
                    "test_bf16_matches_independent_rounding_on_all_decision_boundaries"],
    "coeff_bwd": ["tests/test_coeff_oracle.py"],
}

# (module, text in the oracle, replacement, what the mistake is)
MUTANTS = [
    # bf16 rounding
    ("h_aggregate", "rounded = (u + np.uint64(0x7FFF) + kept_lsb) >> np.uint64(16)",
     "rounded = (u + np.uint64(0x8000)) >> np.uint64(16)", "ties away from zero"),
    ("h_aggregate", "rounded = (u + np.uint64(0x7FFF) + kept_lsb) >> np.uint64(16)",
     "rounded = u >> np.uint64(16)", "truncation instead of rounding"),
    # forward
    ("h_aggregate", """        s01 = np.add(p[0], p[1])
        s23 = np.add(p[2], p[3])
        y = np.add(s01, s23)""",
     """        y = np.add(np.add(np.add(p[0], p[1]), p[2]), p[3])""",
     "left-to-right sum instead of (0+1)+(2+3)"),
    ("h_aggregate", """        s01 = np.add(p[0], p[1])
        s23 = np.add(p[2], p[3])""",
     """        s01 = np.add(p[0], p[2])
        s23 = np.add(p[1], p[3])""", "pairs (0+2)+(1+3)"),
    ("h_aggregate", "        s01 = np.add(p[0], p[1])",
     "        s01 = (pre[:, 0:1].astype(np.float64) * r[:, 0, :] + p[1]).astype(np.float32)",
     "fused multiply-add for the first pair"),
    ("h_aggregate", "        s23 = np.add(p[2], p[3])", "        s23 = p[2]",
     "dropped product"),
    ("h_aggregate", "        p = [np.multiply(pre[:, i:i + 1], r[:, i, :]) for i in range(HC)]",
     "        p = [np.multiply(pre[:, 3 - i:4 - i], r[:, i, :]) for i in range(HC)]",
     "weights applied to the streams in reverse"),
    ("h_aggregate", "quiet = (u >> np.uint64(16)) | np.uint64(0x0040)",
     "quiet = u >> np.uint64(16)", "NaN not quieted (low-payload NaN becomes Inf)"),
    ("h_aggregate", "level = [np.add(level[2 * j], level[2 * j + 1])",
     "level = [np.add(level[j], level[j + len(level) // 2])",
     "strided pairs in the n-stream tree"),
    # backward: grad_residual
    ("h_aggregate", """        prod = np.multiply(pre[:, :, None], g[:, None, :])    # [T,4,H] fp32 RN
    return bf16_rne(prod)""",
     """        prod = np.multiply(widen_bf16(bf16_rne(pre))[:, :, None], g[:, None, :])
    return bf16_rne(prod)""", "pre rounded to bf16 before the product"),
    ("h_aggregate", "        total = np.add(old, prod)                              # fp32 RN",
     "        total = np.add(old, widen_bf16(bf16_rne(prod)))",
     "accumulate rounds the product to bf16 first"),
    # backward: grad_pre order
    ("h_aggregate", "        lane = k % LANES", "        lane = k % 128",
     "groups dealt to 128 lanes"),
    ("h_aggregate", "GROUP = 8\n", "GROUP = 4\n", "groups of 4 elements"),
    ("h_aggregate", "        for j in range(GROUP):", "        for j in reversed(range(GROUP)):",
     "descending order inside a group"),
    ("h_aggregate", "            if h >= H:\n                break",
     "            if h >= H - 1:\n                break", "last element dropped"),
    ("h_aggregate", "                x[..., :off] = np.add(x[..., :off], x[..., off:2 * off])",
     "                x[..., :off] = np.add(x[..., :off], x[..., 2 * off - 1:off - 1:-1])",
     "mirrored pairs in the wave tree"),
    ("h_aggregate", "        return np.add(np.add(y[0], y[2]), np.add(y[1], y[3]))",
     "        return np.add(np.add(y[0], y[1]), np.add(y[2], y[3]))",
     "waves paired (0+1)+(2+3)"),
    ("h_aggregate", "        q = np.multiply(g[:, None, :], r)",
     "        q = np.multiply(g[:, None, :], r[:, ::-1, :])", "streams transposed"),
    # coefficient epilogue
    ("coeff_bwd", "        s = np.divide(post, np.float32(post_scale))", "        s = post",
     "post gate ignores its scale"),
    ("coeff_bwd", "        s = np.divide(post, np.float32(post_scale))",
     "        s = np.multiply(post, np.divide(one, np.float32(post_scale)))",
     "reciprocal of the scale instead of the division"),
    ("coeff_bwd", "np.multiply(pre, np.subtract(one, pre))", "np.multiply(pre, np.add(one, pre))",
     "sign in the sigmoid derivative"),
    ("coeff_bwd", "np.multiply(grad_post, np.multiply(post, np.subtract(one, s)))",
     "np.multiply(grad_post, np.multiply(s, np.subtract(one, s)))",
     "post derivative without its scale"),
    ("coeff_bwd", "CHUNK = 64\n", "CHUNK = 32\n", "32-row chunks"),
    ("coeff_bwd", "acc[:, c % LANES] = np.add(acc[:, c % LANES], P[c])",
     "acc[:, 0] = np.add(acc[:, 0], P[c])", "second stage one sequential chain"),
    ("coeff_bwd", "    off = 32\n    while", "    off = 16\n    while", "tree starts at 16"),
    ("coeff_bwd", "np.array([0] * n + [1] * n", "np.array([1] * n + [0] * n",
     "pre and post groups swapped"),
    ("coeff_bwd", "        prod = np.multiply(d, mix)", "        prod = np.multiply(grad_mix, mix)",
     "alpha gradient from grad_mix instead of d"),
    ("coeff_bwd", "        grad_mix = np.multiply(alpha[k][None, :], d)", "        grad_mix = d.copy()",
     "grad_mix without alpha"),
    ("coeff_bwd", "        for j in range(m):", "        for j in reversed(range(m)):",
     "descending columns in the group sums"),
    ("coeff_bwd", "    grad_b = row_sum(d)", "    grad_b = row_sum(grad_mix)",
     "bias gradient scaled by alpha"),
    ("coeff_bwd", "d_post = np.multiply(grad_post, np.multiply(post,",
     "d_post = np.multiply(grad_post, np.multiply(pre,", "post derivative from the pre gate"),
    ("coeff_bwd", "np.concatenate([d_pre, d_post, grad_res], axis=1)",
     "np.concatenate([d_post, d_pre, grad_res], axis=1)", "pre and post columns swapped"),
    # 16-bit inputs of the coefficient epilogue
    ("coeff_bwd", "            return x.view(np.float16).astype(np.float32)",
     "            return widen_bf16(x)", "fp16 patterns widened as bf16"),
    ("coeff_bwd", "            return x.astype(np.float16).view(np.uint16)",
     "            return widen_bf16(bf16_rne(x)).astype(np.float16).view(np.uint16)",
     "fp16 rounding through bf16 (double rounding)"),
    ("coeff_bwd", "    return narrow(gm, dtype), gb, ga",
     "    return narrow(gm, dtype), widen(narrow(gb, dtype), dtype), ga",
     "bias sums rounded to the input format"),
    ("coeff_bwd", "    gm, gb, ga = coeff_bwd(*rows, alpha, post_scale, n)",
     "    gm, gb, ga = coeff_bwd(*rows[:5], widen(narrow(rows[5], 'bf16'), 'bf16'), alpha, "
     "post_scale, n)", "residual gradient re-rounded to bf16"),
    # the helpers of the fp64 gates
    ("h_aggregate", "    return np.ldexp(1.0, expo - 7)", "    return np.ldexp(1.0, expo - 8)",
     "ulp of a 9-bit significand"),
    ("h_aggregate", "    expo = np.where(v == 0.0, -126, np.maximum(e - 1, -126))",
     "    expo = np.where(v == 0.0, -126, e - 1)", "subnormal ulp not clamped"),
    ("h_aggregate", "    depth = 1 + int(np.log2(n))", "    depth = int(np.log2(n))",
     "error bound without the product's rounding"),
    ("h_aggregate", "    return 0.5 * bf16_ulp(out_bits) + (gamma",
     "    return 1.0 * bf16_ulp(out_bits) + (gamma", "a whole ulp for the output rounding"),
]


def _tree(root: Path, module: str | None = None, before: str = "", after: str = "") -> Path:
    """A copy of oracle/ and the pin files under root, one mutation applied."""
    shutil.copytree(REPO / "oracle", root / "oracle",
                    ignore=shutil.ignore_patterns("__pycache__"))
    (root / "tests").mkdir()
    for name in ("conftest.py", "test_oracle.py", "test_coeff_oracle.py"):
        shutil.copy2(REPO / "tests" / name, root / "tests" / name)
    shutil.copytree(REPO / "tests" / "golden", root / "tests" / "golden")
    os.symlink(REPO / PKG, root / PKG)
    if module is not None:
        path = root / "oracle" / f"{module}.py"
        text = path.read_text()
        path.write_text(text.replace(before, after, 1))
    return root


def _run_pins(root: Path, module: str) -> subprocess.CompletedProcess:
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
           *PINS[module]]
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1", OMP_NUM_THREADS="1")
    return subprocess.run(cmd, cwd=root, env=env, capture_output=True, text=True, timeout=600)


def test_each_mutant_text_occurs_once():
    for module, before, after, why in MUTANTS:
        text = (REPO / "oracle" / f"{module}.py").read_text()
        assert text.count(before) == 1, (module, why)
        assert before != after, why


@pytest.mark.parametrize("module", sorted(PINS))
def test_unchanged_copy_passes_its_pins(tmp_path, module):
    proc = _run_pins(_tree(tmp_path), module)
    assert proc.returncode == 0, proc.stdout[-3000:] + proc.stderr[-3000:]


def test_every_mutant_fails_its_pins(tmp_path):
    def one(k: int):
        module, before, after, why = MUTANTS[k]
        proc = _run_pins(_tree(tmp_path / f"m{k}", module, before, after), module)
        return k, proc

    workers = max(1, min(4, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        results = list(pool.map(one, range(len(MUTANTS))))
    survived, broken = [], []
    for k, proc in results:
        module, _, _, why = MUTANTS[k]
        if proc.returncode == 0:
            survived.append(f"{module}: {why}")
        elif proc.returncode != 1:   # 1 = tests failed; anything else = the run itself broke
            broken.append(f"{module}: {why} (exit {proc.returncode}): {proc.stdout[-500:]}")
    assert not broken, broken
    assert not survived, f"mutants the pins did not catch: {survived}"

"""Build of the gfx950 library (hipcc, in-tree).

Produces, in hyper_connection_residual_mhc_amd/lib/, one shared library per
operation from its source in csrc/ and its public header in include/:

* libmhc_h_aggregate.so  (csrc/mhc_h_aggregate.hip, include/mhc_h_aggregate.h)
* libmhc_coeff_bwd.so    (csrc/mhc_coeff_bwd.hip,   include/mhc_coeff_bwd.h)

The flags fix the arithmetic contract at build time:

* --offload-arch=gfx950           CDNA4 / MI355X code only
* -ffp-contract=off               no multiply-add contraction (the source also
                                  says so with a pragma)
* -Xclang -target-feature -Xclang -packed-fp32-ops
                                  keep the compiler from pairing fp32 lanes
                                  into packed fp32 instructions
* no fast-math (the source refuses to compile under it)

Per library, one performance flag (no effect on any result):

* h_aggregate: -mllvm -amdgpu-kernarg-preload-count=16, so gfx950 loads the
  kernel arguments into scalar registers as each wave starts instead of the
  wave loading them first (its forward runs 14,336 short one-wave blocks at
  T=1024). Measured per call at H=7168: forward 11.76 -> 11.44 us at T=1024
  and 22.62 -> 22.24 us at T=2048, backward 22.08 -> 21.80 us at T=1024;
  about 1% slower at T=128. The coefficient library was 1-3% slower with
  it (few, latency-bound waves), also with its row count moved among the
  preloaded arguments, and builds without it.

`device_asm()` writes the gfx950 assembly of the same source with the same
flags, so tests can scan the machine code this library runs.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import tempfile
from pathlib import Path

PKG_DIR = Path(__file__).resolve().parent
REPO_DIR = PKG_DIR.parent
SRC = PKG_DIR / "csrc" / "mhc_h_aggregate.hip"
COEFF_SRC = PKG_DIR / "csrc" / "mhc_coeff_bwd.hip"
INCLUDE_DIR = REPO_DIR / "include"
HEADER = INCLUDE_DIR / "mhc_h_aggregate.h"
COEFF_HEADER = INCLUDE_DIR / "mhc_coeff_bwd.h"
LIB_DIR = PKG_DIR / "lib"
LIB_PATH = LIB_DIR / "libmhc_h_aggregate.so"
COEFF_LIB_PATH = LIB_DIR / "libmhc_coeff_bwd.so"
BUILD_DIR = REPO_DIR / "_build"

# source -> library, header
LIBRARIES = {SRC: (LIB_PATH, HEADER), COEFF_SRC: (COEFF_LIB_PATH, COEFF_HEADER)}
# source -> its own flags (see the module docstring)
SOURCE_FLAGS = {SRC: ["-mllvm", "-amdgpu-kernarg-preload-count=16"], COEFF_SRC: []}

ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-I", str(INCLUDE_DIR),
]


def hipcc() -> str:
    path = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not Path(path).exists():
        raise RuntimeError(f"hipcc not found (looked for {path})")
    return path


def _run(cmd: list[str]) -> None:
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that
    # warning is expected and harmless.
    lines = [ln for ln in proc.stdout.splitlines()
             if "packed-fp32-ops" not in ln and "--hip-link" not in ln]
    if proc.returncode != 0:
        raise RuntimeError("build failed:\n$ " + " ".join(cmd) + "\n" + "\n".join(lines))
    if lines:
        print("\n".join(lines))


def _build_one(src: Path, lib: Path, extra_flags: list[str] | None) -> Path:
    LIB_DIR.mkdir(parents=True, exist_ok=True)
    fd, tmp = tempfile.mkstemp(prefix=f".{lib.stem}.", suffix=".so.tmp", dir=LIB_DIR)
    os.close(fd)
    try:
        cmd = [hipcc(), *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), "-fPIC", "-shared",
               *(extra_flags or []), str(src), "-o", tmp]
        _run(cmd)
        os.replace(tmp, lib)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return lib


def build_library(extra_flags: list[str] | None = None) -> Path:
    """Compile every shared library (always recompiles); returns the
    h_aggregate library's path."""
    for src, (lib, _) in LIBRARIES.items():
        _build_one(src, lib, extra_flags)
    return LIB_PATH


def device_asm(out: Path | None = None, extra_flags: list[str] | None = None,
               src: Path = SRC) -> Path:
    """Write the gfx950 assembly of one library source (same flags)."""
    BUILD_DIR.mkdir(parents=True, exist_ok=True)
    out = Path(out) if out else BUILD_DIR / f"{src.stem}-{ARCH}.s"
    cmd = [hipcc(), *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), "--cuda-device-only", "-S",
           *(extra_flags or []), str(src), "-o", str(out)]
    _run(cmd)
    return out


def library_is_built() -> bool:
    return all(lib.exists() for lib, _ in LIBRARIES.values())


if __name__ == "__main__":
    print(build_library())

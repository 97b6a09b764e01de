"""Build of the gfx950 library (hipcc, in-tree).

Produces hyper_connection_residual_mhc_amd/lib/libmhc_h_aggregate.so from
csrc/mhc_h_aggregate.hip and the public header in include/. The flags fix the
arithmetic contract at build time:

* --offload-arch=gfx950           CDNA4 / MI355X code only
* -ffp-contract=off               no multiply-add contraction (the source also
                                  says so with a pragma)
* -Xclang -target-feature -Xclang -packed-fp32-ops
                                  keep the compiler from pairing fp32 lanes
                                  into packed fp32 instructions
* no fast-math (the source refuses to compile under it)

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
INCLUDE_DIR = REPO_DIR / "include"
HEADER = INCLUDE_DIR / "mhc_h_aggregate.h"
LIB_DIR = PKG_DIR / "lib"
LIB_PATH = LIB_DIR / "libmhc_h_aggregate.so"
BUILD_DIR = REPO_DIR / "_build"

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


def build_library(extra_flags: list[str] | None = None) -> Path:
    """Compile the shared library; returns its path. Always recompiles."""
    LIB_DIR.mkdir(parents=True, exist_ok=True)
    fd, tmp = tempfile.mkstemp(prefix=".libmhc_h_aggregate.", suffix=".so.tmp", dir=LIB_DIR)
    os.close(fd)
    try:
        cmd = [hipcc(), *COMMON_FLAGS, "-fPIC", "-shared", *(extra_flags or []),
               str(SRC), "-o", tmp]
        _run(cmd)
        os.replace(tmp, LIB_PATH)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return LIB_PATH


def device_asm(out: Path | None = None, extra_flags: list[str] | None = None) -> Path:
    """Write the gfx950 assembly of the library source (same flags)."""
    BUILD_DIR.mkdir(parents=True, exist_ok=True)
    out = Path(out) if out else BUILD_DIR / f"mhc_h_aggregate-{ARCH}.s"
    cmd = [hipcc(), *COMMON_FLAGS, "--cuda-device-only", "-S", *(extra_flags or []),
           str(SRC), "-o", str(out)]
    _run(cmd)
    return out


def library_is_built() -> bool:
    return LIB_PATH.exists()


if __name__ == "__main__":
    print(build_library())

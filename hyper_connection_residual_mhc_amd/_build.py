"""Build of the gfx950 library (hipcc, in-tree).

Produces, in hyper_connection_residual_mhc_amd/lib/, one shared library per
operation from its source in csrc/ and its public header in include/, plus
the measurement library the tests and the benchmark use:

* libmhc_h_aggregate.so  (csrc/mhc_h_aggregate.hip, include/mhc_h_aggregate.h)
* libmhc_coeff_bwd.so    (csrc/mhc_coeff_bwd.hip,   include/mhc_coeff_bwd.h)
* libmhc_probes.so       (csrc/mhc_probes.hip,      csrc/mhc_probes.h;
                          not part of the operation)

Beside each library, `<library>.build.json` records a digest of what built
it: its source, every header in csrc/ and include/, the flags and the
target. The loaders (_lib) refuse a library whose digest no longer matches
the sources in the tree, so a stale binary is never run by mistake;
`ensure_built()` (used by the tests, the smoke check and the benchmark)
builds when a library is missing or stale.

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

import hashlib
import json
import os
import shutil
import subprocess
import tempfile
from pathlib import Path

PKG_DIR = Path(__file__).resolve().parent
REPO_DIR = PKG_DIR.parent
SRC = PKG_DIR / "csrc" / "mhc_h_aggregate.hip"
COEFF_SRC = PKG_DIR / "csrc" / "mhc_coeff_bwd.hip"
PROBE_SRC = PKG_DIR / "csrc" / "mhc_probes.hip"
INCLUDE_DIR = REPO_DIR / "include"
HEADER = INCLUDE_DIR / "mhc_h_aggregate.h"
COEFF_HEADER = INCLUDE_DIR / "mhc_coeff_bwd.h"
LIB_DIR = PKG_DIR / "lib"
LIB_PATH = LIB_DIR / "libmhc_h_aggregate.so"
COEFF_LIB_PATH = LIB_DIR / "libmhc_coeff_bwd.so"
PROBE_LIB_PATH = LIB_DIR / "libmhc_probes.so"
BUILD_DIR = REPO_DIR / "_build"

# source -> library, header
LIBRARIES = {SRC: (LIB_PATH, HEADER), COEFF_SRC: (COEFF_LIB_PATH, COEFF_HEADER),
             PROBE_SRC: (PROBE_LIB_PATH, PKG_DIR / "csrc" / "mhc_probes.h")}
# source -> its own flags (see the module docstring)
SOURCE_FLAGS = {SRC: ["-mllvm", "-amdgpu-kernarg-preload-count=16"], COEFF_SRC: [],
                PROBE_SRC: []}

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


def build_info_path(lib: Path) -> Path:
    return lib.with_name(lib.name + ".build.json")


def source_digest(src: Path, extra_flags: list[str] | None = None) -> str:
    """sha256 over what a library is built from: its source file, every
    header in csrc/ and include/ (by name and content), the compile flags
    (the include path by its place in the repository, not its absolute path)
    and the target."""
    h = hashlib.sha256()
    h.update(src.name.encode() + b"\0" + src.read_bytes())
    for hdr in sorted(list((PKG_DIR / "csrc").glob("*.h")) + list(INCLUDE_DIR.glob("*.h"))):
        h.update(hdr.relative_to(REPO_DIR).as_posix().encode() + b"\0" + hdr.read_bytes())
    flags = [f if f != str(INCLUDE_DIR) else "<repo>/include" for f in COMMON_FLAGS]
    flags += SOURCE_FLAGS.get(src, []) + list(extra_flags or [])
    h.update(json.dumps({"flags": flags, "arch": ARCH}).encode())
    return h.hexdigest()


def recorded_digest(lib: Path) -> str | None:
    """The digest stored beside a built library, or None."""
    try:
        return json.loads(build_info_path(lib).read_text()).get("source_digest")
    except (OSError, ValueError):
        return None


def _build_one(src: Path, lib: Path, extra_flags: list[str] | None) -> Path:
    LIB_DIR.mkdir(parents=True, exist_ok=True)
    fd, tmp = tempfile.mkstemp(prefix=f".{lib.stem}.", suffix=".so.tmp", dir=LIB_DIR)
    os.close(fd)
    info = build_info_path(lib)
    try:
        cmd = [hipcc(), *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), "-fPIC", "-shared",
               *(extra_flags or []), str(src), "-o", tmp]
        _run(cmd)
        if info.exists():
            info.unlink()  # never leave a record that describes another binary
        os.replace(tmp, lib)
        info.write_text(json.dumps({"source": src.name,
                                    "source_digest": source_digest(src, extra_flags)}) + "\n")
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
    """Every library exists and was built from the sources now in the tree."""
    return all(lib.exists() and recorded_digest(lib) == source_digest(src)
               for src, (lib, _) in LIBRARIES.items())


def ensure_built() -> None:
    """Build when a library is missing or was built from other sources."""
    if not library_is_built():
        stale = [lib.name for src, (lib, _) in LIBRARIES.items()
                 if lib.exists() and recorded_digest(lib) != source_digest(src)]
        if stale:
            print(f"rebuilding: {', '.join(stale)} built from other sources", flush=True)
        build_library()


if __name__ == "__main__":
    print(build_library())

"""Build step for the HIP libraries (gfx950, in-tree): libidx_paged_mqa.so, the
indexer, and libidx_read_stream.so, the bare key-page read stream that the
benchmark measures as the reachable HBM read rate."""
from __future__ import annotations

import os
import shutil
import subprocess
from pathlib import Path

PKG_DIR = Path(__file__).resolve().parent
REPO_DIR = PKG_DIR.parent
SOURCES = [PKG_DIR / "csrc" / "paged_mqa_logits.hip"]
LIB_PATH = PKG_DIR / "libidx_paged_mqa.so"
STREAM_SOURCES = [PKG_DIR / "csrc" / "read_stream.hip"]
STREAM_LIB_PATH = PKG_DIR / "libidx_read_stream.so"
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build_command(out: Path = LIB_PATH, sources=None) -> list[str]:
    return [
        hipcc(),
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-shared",
        "-fPIC",
        # packed fp32 VALU ops are kept out of every kernel
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{REPO_DIR / 'include'}",
        *[str(s) for s in (SOURCES if sources is None else sources)],
        "-o", str(out),
    ]


def build(verbose: bool = False) -> Path:
    """Compile both libraries; always recompiles.  Writes atomically."""
    _compile(STREAM_LIB_PATH, STREAM_SOURCES, verbose)
    return _compile(LIB_PATH, SOURCES, verbose)


def _compile(lib: Path, sources, verbose: bool) -> Path:
    tmp = lib.with_name(lib.name + ".tmp")
    cmd = build_command(tmp, sources)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or res.returncode != 0:
        out = (res.stdout + res.stderr).strip()
        # hipcc's host pass does not know the packed-fp32 feature; drop that noise
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if out:
            print(out)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))

"""Build the HIP library libattn_gfx950.so in-tree with hipcc (gfx950 only)."""
from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
LIB = PKG / "libattn_gfx950.so"
SOURCES = ["attn_api.hip", "prefill_gfx950.hip", "paged_gfx950.hip", "append_gfx950.hip", "bwd_gfx950.hip",
           "check_gfx950.hip", "noalloc_gfx950.hip"]
HEADERS = ["attn_internal.h", "append_internal.h", "bwd_internal.h", "attn_mfma_core.h", "attn_mfma_kernel.h",
           "attn_mfma_pipe.h", "check_internal.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # kernels never rely on NaN propagation (masked slots are selected away by
    # index), which lets fmaxf lower to v_max3_f32 without operand quieting
    "-Xarch_device", "-fno-honor-nans",
]


def build(verbose: bool = False, out: Path | None = None, extra_flags=()) -> Path:
    """Compile every HIP source into one shared library (always recompiles)."""
    out = Path(out) if out else LIB
    tmp = out.with_suffix(".so.tmp%d" % os.getpid())
    cmd = [HIPCC, *FLAGS, *extra_flags, "-I", str(CSRC), "-I", str(PKG.parent / "include"),
           *[str(CSRC / s) for s in SOURCES], "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed (%d)" % res.returncode)
    os.replace(tmp, out)
    return out


def is_stale(lib: Path = LIB) -> bool:
    if not lib.exists():
        return True
    t = lib.stat().st_mtime
    deps = [CSRC / s for s in SOURCES + HEADERS] + [PKG.parent / "include" / "attn.h"]
    return any(p.stat().st_mtime > t for p in deps if p.exists())


if __name__ == "__main__":
    print(build(verbose=True))

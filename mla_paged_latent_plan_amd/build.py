"""Build libmla.so (the HIP kernels and the C ABI of include/mla.h) in-tree for gfx950."""

from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libmla.so")
SOURCES = ["plan.hip", "decode.hip", "combine.hip", "kvwrite.hip", "absorb.hip", "swa_runs.hip", "gather.hip", "sparse_meta.hip", "check.hip", "api.hip"]
HEADERS = ["mla_internal.h", "layer_internal.h"]
PUBLIC_HEADER = os.path.join(os.path.dirname(PKG_DIR), "include", "mla.h")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libmla.so")
    return path


def source_id() -> str:
    """16 hex digits of the SHA-256 of every source the library is built from (the HIP sources,
    internal headers and include/mla.h, in a fixed order). The build embeds it in libmla.so, where
    mla_build_id() returns it, so a loaded library can be matched with the sources beside it."""
    h = hashlib.sha256()
    for path in [os.path.join(CSRC, f) for f in SOURCES + HEADERS] + [PUBLIC_HEADER]:
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libmla.so next to this file; returns the library path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, f'-DMLA_BUILD_ID="{source_id()}"', *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in proc.stderr.splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))

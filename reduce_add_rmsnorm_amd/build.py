"""Build step for libsprms.so (HIP, gfx950), in-tree next to this file.

    python -m reduce_add_rmsnorm_amd.build
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
# the fused shard kernel, the layout kernels (gather, regroupings), the
# producer GEMM, and the host-only C ABI helpers
SRCS = [os.path.join(PKG, "csrc", f) for f in ("sprms.hip", "layout.hip", "gemm.hip", "abi.cpp")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsprms.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -O3 without fast-math: the fp32 add order of the source is kept.
# packed-fp32-ops is disabled for every HIP compile in this project.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build_library(verbose: bool = False) -> str:
    """Compile csrc/*.hip into libsprms.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *HIPCC_FLAGS, "-I", INCLUDE, "-o", tmp, *SRCS]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"  # the host pass does not know this GPU feature
    msgs = [ln for ln in (proc.stderr or "").splitlines() if noise not in ln and "--hip-link" not in ln]
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))

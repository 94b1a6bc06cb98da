"""Build libsige.so (HIP, gfx950) in-tree, next to this file.

    python -m spatially_sparse_incremental_amd.build [-v]

Every HIP source is compiled for gfx950 only.  Packed fp32 instructions are
switched off for the device code (`-Xclang -target-feature -Xclang
-packed-fp32-ops`); hipcc's host pass warns that it does not know that
feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["sige_api.hip", "kernels_mask.hip", "kernels_conv.hip", "kernels_layer.hip", "kernels_attn.hip"]
LIB = os.path.join(PKG, "libsige.so")


def hipcc_command(out: str) -> list[str]:
    return ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            "-o", out] + [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in (r.stderr or "").splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

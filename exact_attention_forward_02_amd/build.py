"""Compile the gfx950 HIP library in-tree (hipcc cross-compiles without a GPU)."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libattn_fwd.so")
SOURCES = [os.path.join(CSRC, "attn_fwd_kernel.hip"), os.path.join(CSRC, "attn_merge_kernel.hip"),
           os.path.join(CSRC, "attn_bwd_kernel.hip"), os.path.join(CSRC, "attn_decode_kernel.hip"),
           os.path.join(CSRC, "attn_api.cpp")]
ARCH = "gfx950"

# Packed fp32 VALU forms are kept out of the generated code.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build(output: str = LIBRARY, extra_flags=()) -> str:
    """Build libattn_fwd.so and return its path (always recompiles)."""
    tmp = output + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-o", tmp, *SOURCES]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build())

"""Build libpkv.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m paged_kv_cache_26_amd.build  (or call build()).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libpkv.so")
SOURCES = ["pkv_capi.hip", "pkv_append.hip", "pkv_decode.hip", "pkv_block_manager.hip",
           "pkv_measure.hip"]
ARCH = "gfx950"

# Packed-fp32 instructions are disabled on purpose: every fp32 operation in the kernels
# is written as scalar float code and must lower to unpacked VALU instructions.
# Matrix-core accumulators are kept in ordinary vector registers (the MFMA VGPR form):
# the kernels that accumulate P.V on the matrix cores (multi-query, quantized, shared-
# prefix pass) otherwise shuttle them through the accumulation registers around every
# rescale, which costs 3-10% in those kernels; the other kernels compile the same.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libpkv)")


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libpkv.so next to this file; return its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, f"-I{os.path.join(ROOT, 'include')}",
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (proc.stdout + proc.stderr).splitlines() if noise not in ln]
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)

"""Build libpkv.so (HIP, gfx950) in-tree with hipcc.

Every translation unit is compiled to an object in parallel (the decode kernels once per
dtype), then the objects are linked into paged_kv_cache_26_amd/libpkv.so.

Usage: python -m paged_kv_cache_26_amd.build  (or call build()).
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
OBJ_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libpkv.so")
ARCH = "gfx950"

# (object name, source, extra flags). Host C++ (*.cpp) holds the C ABI, the dtype dispatch
# and the block manager; the kernels are in *.hip. pkv_decode.hip holds every decode,
# and merge kernel (with the shared-prefix tasks) and is compiled once per dtype.
UNITS = [
    ("pkv_capi", "pkv_capi.cpp", []),
    ("pkv_dispatch", "pkv_dispatch.cpp", []),
    ("pkv_block_manager", "pkv_block_manager.cpp", []),
    ("pkv_append", "pkv_append.hip", []),
    ("pkv_measure", "pkv_measure.hip", []),
    ("pkv_scratch", "pkv_scratch.hip", []),
    ("pkv_decode_f32", "pkv_decode.hip", ["-DPKV_DECODE_DTYPE=0"]),
    ("pkv_decode_f16", "pkv_decode.hip", ["-DPKV_DECODE_DTYPE=1"]),
    ("pkv_decode_bf16", "pkv_decode.hip", ["-DPKV_DECODE_DTYPE=2"]),
]
SOURCES = sorted({src for _, src, _ in UNITS})

# Packed-fp32 instructions are disabled on purpose: every fp32 operation in the kernels
# is written as scalar float code and must lower to unpacked VALU instructions.
# Matrix-core accumulators are kept in ordinary vector registers (the MFMA VGPR form):
# the kernels that accumulate P.V on the matrix cores (multi-query, quantized, shared-
# prefix tasks) otherwise shuttle them through the accumulation registers around every
# rescale, which costs 3-10% in those kernels; the other kernels compile the same.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]
# hipcc's host pass does not know the packed-fp32 feature and says so; that line is dropped
_NOISE = "'-packed-fp32-ops' is not a recognized feature"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libpkv)")


def _run(cmd: list[str]) -> tuple[int, list[str]]:
    proc = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (proc.stdout + proc.stderr).splitlines() if _NOISE not in ln]
    return proc.returncode, msgs


def _jobs() -> int:
    try:
        cpus = len(os.sched_getaffinity(0))
    except AttributeError:
        cpus = os.cpu_count() or 1
    return max(1, min(cpus, len(UNITS), int(os.environ.get("MAX_JOBS", "16"))))


def build(verbose: bool = False) -> str:
    """Compile every translation unit and link libpkv.so next to this file; return its path."""
    cc = hipcc()
    os.makedirs(OBJ_DIR, exist_ok=True)
    inc = f"-I{os.path.join(ROOT, 'include')}"

    def compile_unit(unit):
        name, src, extra = unit
        obj = os.path.join(OBJ_DIR, name + ".o")
        cmd = [cc, *HIP_FLAGS, *extra, inc, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        rc, msgs = _run(cmd)
        return name, obj, rc, msgs

    with concurrent.futures.ThreadPoolExecutor(_jobs()) as pool:
        results = list(pool.map(compile_unit, UNITS))
    failed = [(n, m) for n, _, rc, m in results if rc != 0]
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(
            f"[{n}]\n" + "\n".join(m) for n, m in failed))
    if verbose:
        for n, _, _, m in results:
            if m:
                print(f"[{n}]\n" + "\n".join(m), flush=True)
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for _, o, _, _ in results],
           "-o", tmp]
    rc, msgs = _run(cmd)
    if rc != 0:
        raise RuntimeError("link failed:\n" + "\n".join(msgs))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:]))
    sys.exit(0)

"""Build libpq2.so (the gfx950 HIP kernels and their C ABI) in-tree.

    python gemm_int8_act_amd/build.py

(run it as a script: importing the package would load the library it builds).

Each .hip source compiles to an object in parallel, then hipcc links the
shared library next to this file.  Packed-FP32 instruction selection is
switched off for the device code (-target-feature -packed-fp32-ops).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpq2.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["api.hip", "quantize.hip", "small_m.hip", "small_m_wg.hip", "tiles.hip", "prefill.hip", "probe.hip"]
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: a ROCm toolchain is needed to build libpq2")
    return path


# Per-source extra flags.  The prefill kernel rescales every MFMA result on
# the vector ALU; asking the backend for the VGPR form of the MFMA keeps the
# accumulators out of AGPRs and saves one register move per output and group.
EXTRA_FLAGS = {
    "prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libpq2.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    workers = min(len(SOURCES), max(1, (os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as pool:
        objs = list(pool.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

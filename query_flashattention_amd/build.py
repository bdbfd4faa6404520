"""Build step for libds4attn.so: hipcc, gfx950 only, in-tree.

Each HIP source is compiled to an object in ``_build/`` (in parallel), then the
objects are linked into ``query_flashattention_amd/libds4attn.so``.  The library
is replaced atomically so a running process never sees a half-written file.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libds4attn.so")
PROBES_LIB = os.path.join(PKG, "libds4probes.so")
ARCH = "gfx950"

# Packed fp32 instructions stay off: only scalar/vector fp32 code is emitted.
# MFMA accumulators are allocated in ordinary VGPRs: the attention kernels keep
# the output tile across the key loop and rescale it with vector ALU code, which
# would otherwise shuttle it between AGPRs and VGPRs on every iteration.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-mcode-object-version=5",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form=1",
          "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libds4attn")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source under csrc/ for gfx950 and link libds4attn.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-mcode-object-version=5", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    build_probes(verbose)
    return LIB


def build_probes(verbose: bool = False) -> str:
    """The measurement probes (achievable HBM read bandwidth and MFMA throughput)
    as their own library, libds4probes.so; only the benchmark loads it."""
    src = os.path.join(PKG, "probes", "peaks.hip")
    tmp = PROBES_LIB + ".tmp"
    cmd = [hipcc(), *COMMON, "-shared", src, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, PROBES_LIB)
    if verbose:
        print(f"built {PROBES_LIB}")
    return PROBES_LIB


if __name__ == "__main__":
    build(verbose=True)

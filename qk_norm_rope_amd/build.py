"""Build libqknr.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: python -m qk_norm_rope_amd.build   (or call build()).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libqknr.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

ARCH = "gfx950"
# Packed float32 instructions are kept out of every kernel.
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"),
]
SOURCES = {
    # The append kernel's float32 arithmetic must not be contracted into FMAs:
    # its stored bytes are specified operation by operation.
    "append.hip": ["-ffp-contract=off"],
    # MFMA accumulators in VGPRs: the small-batch decode kernel otherwise takes 4
    # AGPRs on top of 126 VGPRs, which leaves room for 3 workgroups per CU instead of 4
    "decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
    "prefill.hip": [],
    "generic.hip": [],
    "step.hip": [],
    "check.hip": [],
    "probe.hip": [],
    "api.cpp": ["-ffp-contract=off"],
}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libqknr")
    return path


def _compile(src: str, extra: list) -> str:
    obj = os.path.join(BUILD_DIR, src + ".o")
    cmd = [hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libqknr.so next to this file; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda kv: _compile(*kv), SOURCES.items()))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

"""Builds ``libsi_indexer.so`` (the HIP kernels and the C ABI) in-tree for gfx950.

    python streaming_top_selection_amd/build.py   (run by path: importing the package
                                                  loads the library it builds)

Every ``csrc/*.hip`` source is compiled with hipcc to an object in parallel, then the
objects are linked into ``streaming_top_selection_amd/libsi_indexer.so``.
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsi_indexer.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    # inputs are finite (non-finite values are outside the ABI contract), so max(z, 0)
    # needs no NaN quieting: one v_max_f32 per element
    "-fno-honor-nans",
    # packed fp32 VALU ops stay off: every fp32 op is an ordinary v_*_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results and accumulators in VGPRs: the epilogue reads every MFMA result
    # with VALU ops, which cannot read AGPRs (the AGPRs then hold the key operands)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall",
    "-Wno-unused-function",
    f"-I{INCLUDE}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    # the largest units (the KB = 4 select kernels) first, so the pool stays busy
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")),
                     key=lambda f: (not ("kt512" in f or "kt1024" in f), f))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, jobs=int(sys.argv[1]) if len(sys.argv) > 1 else 8)

"""Builds ``libsi_indexer.so`` (the HIP kernels and the C ABI) in-tree for gfx950.

    python streaming_top_selection_amd/build.py   (run by path: importing the package
                                                  loads the library it builds)

Every ``csrc/*.hip`` source is compiled with hipcc to an object in parallel (the
select kernel's instantiation file once per register-tile shape and operand mode),
then the objects are linked into ``streaming_top_selection_amd/libsi_indexer.so``.
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


# Select kernel register-tile shapes (waves, key blocks per wave, register tiles per key
# tile), one per key tile 64, 128, 256, 512, 768, 1024 (the plan's table), and the
# operand modes (bf16 x bf16, bf16 x E4M3, E4M3 x E4M3, E4M3 x MXFP4).  Each pair is
# its own object of si_select_inst.hip.
SELECT_SHAPES = [(2, 1, 1), (4, 1, 1), (4, 2, 1), (4, 4, 1), (4, 2, 3), (4, 4, 2)]
SELECT_OPS = [0, 1, 2, 3]
SELECT_INST = "si_select_inst.hip"


def _compile(job) -> str:
    src, defs, tag = job
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + tag + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *defs, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src} {defs}:\n{r.stdout}\n{r.stderr}")
    return obj


def jobs_list():
    """(source, -D flags, object tag) of every object of the library."""
    out = []
    for nw, kb, ns in SELECT_SHAPES:
        for op in SELECT_OPS:
            out.append((os.path.join(CSRC, SELECT_INST),
                        [f"-DSI_NW={nw}", f"-DSI_KB={kb}", f"-DSI_NS={ns}", f"-DSI_OP={op}"],
                        f".{nw}_{kb}_{ns}_op{op}"))
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        if os.path.basename(src) != SELECT_INST:
            out.append((src, [], ""))
    # the largest units (four key blocks per wave) first, so the pool stays busy
    return sorted(out, key=lambda j: (not any(d in ("-DSI_KB=4",) for d in j[1]), j[2]))


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, jobs_list()))
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

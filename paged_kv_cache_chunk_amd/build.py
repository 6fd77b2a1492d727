"""Build libpkv.so (hipcc, gfx950) in-tree.

    python -m paged_kv_cache_chunk_amd.build

Compiles every csrc/*.hip and csrc/*.cpp to an object under _build/ and links
them into paged_kv_cache_chunk_amd/libpkv.so.  Always recompiles.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libpkv.so")
BUILD = os.path.join(PKG, "_build")

ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Per-source machine-scheduler strategy of the LLVM AMDGPU backend, chosen by
# measurement on MI355X: the dK/dV and forward kernels (one or two waves per
# SIMD, register-bound) gain from the iterative ILP scheduler, which hoists LDS
# reads ahead of the MFMAs that consume them; the dQ kernel from the max-ILP one.
# dK/dV also takes MFMA results in VGPRs (its K/V operands are pinned to
# AGPRs in the source), so the softmax reads S and dP without AGPR copies.
SOURCE_FLAGS = {
    "attn_bf16_dkdv.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp",
                           "-mllvm", "-amdgpu-mfma-vgpr-form"],
    "attn_bf16_fwd.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
    "attn_bf16_dq.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libpkv)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *SOURCE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    workers = max(1, min(len(srcs), os.cpu_count() or 1, 16))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT} from {len(srcs)} sources", file=sys.stderr)
    return OUT


if __name__ == "__main__":
    build()

"""Builds the HIP library ``libmla_pcp.so`` in-tree for gfx950 with hipcc.

Every translation unit is compiled to an object under ``_build/`` (in parallel), then
linked into ``context_mla_prefill_amd/libmla_pcp.so``. Packed-fp32 instruction
selection is disabled for device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmla_pcp.so")

SOURCES = ["api.hip", "partition.hip", "kv_insert.hip", "merge.hip", "attn_dense.hip", "attn_dense_wide.hip",
           "attn_sparse_wide.hip", "topk_select.hip", "split_plan.hip"]

# Per-file flags. The attention kernels' builtin MFMAs accumulate in VGPRs (MFMA VGPR form):
# the scores everywhere, and O in the 64-row kernels, whose rare rescale is then plain VALU
# work while Q sits in AGPRs; the wide kernels (512 + 64 dense, sparse) keep O
# in AGPRs through inline-asm P V MFMAs instead.
EXTRA = {"attn_dense.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "attn_dense_wide.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "attn_sparse_wide.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []

    def one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        _run(cmd)
        return obj

    with ThreadPoolExecutor(min(jobs, len(SOURCES))) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Build librra.so in-tree with hipcc for gfx950.

    python -m dynamic_block_sparse_sample_amd.build [-j N]

Every HIP source is compiled to an object under _build/ (in parallel), then
linked into dynamic_block_sparse_sample_amd/librra.so.  Always rebuilds.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librra.so")

SOURCES = [
    "rra_validate.cpp",
    "rra_api.cpp",
    "kernels/cast.hip",
    "kernels/stride_aggregate.hip",
    "kernels/block_scores.hip",
    "kernels/top_tau.hip",
    "kernels/block_mass.hip",
    "kernels/xattn_scores.hip",
    "kernels/flash_attn.hip",
    "rra_noalloc.hip",
]

ARCH = "gfx950"
# Packed-FP32 VALU forms are disabled for all device code.
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics"]
# Per-file additions: MFMA results in VGPRs rather than AGPRs.  block_scores:
# the softmax and pooling read them without v_accvgpr_read copies (16 per tile
# and pass; the kernel is VALU-bound: 9 % faster at 128K, same bits).
# flash_attn: the 128-query kernels compile to the same code; the 64-query ones
# no longer shuttle O through AGPRs (<128,64>: 380 -> 262 registers).
_VGPR_MFMA = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
FILE_FLAGS = {"kernels/block_scores.hip": _VGPR_MFMA, "kernels/flash_attn.hip": _VGPR_MFMA}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build librra.so")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace("/", "_") + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [hipcc(), *COMMON, *HIP_FLAGS, *FILE_FLAGS.get(src, []), "-x", "hip", "-c", path, "-o", obj]
    else:
        cmd = [hipcc(), *COMMON, "-c", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    _link(objs, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=None)
    args = ap.parse_args(argv)
    build(args.j, verbose=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

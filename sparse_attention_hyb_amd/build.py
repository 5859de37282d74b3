"""Build libhyb.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m sparse_attention_hyb_amd.build [--jobs N]

Objects go to ``_build/`` at the repository root; the shared library is written next to this
file so that the binding (and every GPU run that receives the source tree) finds it.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libhyb.so")

SOURCES = ["hyb_api.cpp", "compress.hip", "index_score.hip", "topk.hip", "attn.hip", "hbm_probe.hip",
           "offload.hip"]
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
# The attention kernel keeps 128 output accumulators live across the softmax rescale. With the
# default heuristic the backend parks them in AGPRs and copies all of them to VGPRs and back on
# every key tile (about 800 v_accvgpr moves per tile loop); forcing the VGPR form of the MFMAs
# removes those moves (register use drops from 507 to 365, no spills). The indexer's score tiles
# end in a ReLU-weighted head sum on the VALU: in AGPRs their 32 accumulators took 32
# v_accvgpr_read per tile and key block (fp4 keys: about a fifth of the loop's VALU work).
_VGPR_MFMA = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
EXTRA = {"attn.hip": _VGPR_MFMA, "index_score.hip": _VGPR_MFMA}


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libhyb.so)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + FLAGS + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(jobs: int = 8, verbose: bool = False) -> str:
    """Compile every source and link libhyb.so. Always rebuilds. Returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking libhyb.so failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    args = ap.parse_args()
    try:
        build(args.jobs, verbose=True)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)

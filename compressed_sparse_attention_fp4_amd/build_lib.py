"""Build libcsa2.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

Usage: python -m compressed_sparse_attention_fp4_amd.build_lib
Every call recompiles.  Objects go to _build/ (git-ignored); the library lands next to
this file, where the binding loads it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libcsa2.so")
BUILD = os.path.join(ROOT, "_build", "csa2")

SOURCES = ["csa2_api.cpp", "k_tail_quant.hip", "k_score.hip", "k_topk.hip", "k_attn.hip", "k_produce.hip", "k_fused.hip",
           "k_check.hip"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libcsa2.so)")


COMMON = [
    "-std=c++17", "-O3", "-fPIC", "--offload-arch=gfx950",
    # packed fp32 VALU ops stay off: the compiler may not form v_pk_{add,mul,fma}_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"),
]


# Per-source flags.  The index-score kernels consume every MFMA result with VALU
# arithmetic at once, so their MFMAs write VGPRs (no AGPR round trip).  They also schedule
# for instruction-level parallelism: the fused pool scoring + top-k 1.5-2% faster, prefill
# scoring (row pairs) 1.5-2% faster, decode scoring unchanged; the attention kernel was
# slower under it.
EXTRA = {"k_score.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-mllvm", "-amdgpu-sched-strategy=max-ilp"],
         "k_fused.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp", "-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = [] if src.endswith(".hip") else ["-x", "hip"]
    cmd = [hipcc()] + COMMON + EXTRA.get(src, []) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr[-6000:]))
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr[-4000:]))
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build()
    sys.exit(0)

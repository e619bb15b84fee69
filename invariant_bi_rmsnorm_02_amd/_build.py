"""Build libbi.so and libbi_adaptive.so (HIP for gfx950) in-tree with hipcc.

libbi_adaptive.so holds the shape-adaptive comparators (include/bi_adaptive.h)
and the two libbi kernels they fall back to (GEMM, RMSNorm); nothing in
libbi.so depends on it.

Every translation unit is compiled with -ffp-contract=off and without fast
math, so each floating-point expression runs exactly as written (the
batch-invariance rules depend on it), and with packed-fp32 instruction
generation disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libbi.so")
ADAPTIVE_LIB = os.path.join(PKG, "libbi_adaptive.so")
ADAPTIVE_SOURCES = ["adaptive.hip"]
ADAPTIVE_SHARED = ["gemm.hip", "rmsnorm.hip"]   # libbi objects linked into the comparator library
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["api.cpp", "rmsnorm.hip", "gemm.hip", "gemm_fused.hip", "kv_append.hip", "attn_decode.hip",
           "attn_prefill.hip", "log_softmax.hip", "moe.hip", "lm_head.hip", "pointwise.hip", "scratch.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# -amdgpu-mfma-vgpr-form: MFMA accumulators in VGPRs rather than AGPRs, so the
# VALU can rescale them in place (the attention accumulators are rescaled on
# every 32-key step; in AGPRs each rescale costs two moves per element).  It
# selects register classes only, never instructions or their order.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
         "-fno-fast-math", "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form", "-I", INCLUDE, "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + ADAPTIVE_SOURCES
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in ADAPTIVE_SOURCES + ADAPTIVE_SHARED], ADAPTIVE_LIB)
    if verbose:
        print(f"built {LIB} and {ADAPTIVE_LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)

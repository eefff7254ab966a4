"""Build libdsa.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

Usage: python -m sparse_attention_amd.build_lib   (or build() from Python).
Every source is compiled for gfx950 only; packed-fp32 instructions are
disabled for device code (-packed-fp32-ops).
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdsa.so")

HIP_SOURCES = ["score_decode.hip", "score_decode_heads.hip", "score_prefill.hip", "topk.hip", "sparse_attn.hip",
               "sparse_attn_decode.hip", "sparse_attn_wide.hip", "cache_write.hip", "score_prefill_fold.hip", "decode_static.hip",
               "attn_masked_dense.hip"]
CPP_SOURCES = ["dsa_api.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source device options.  The decode attention kernel keeps its
# 128-register output accumulator in VGPRs (MFMA results written to VGPRs,
# read-only MFMA operands free to live in AGPRs); otherwise the compiler
# copies the whole accumulator between AGPRs and VGPRs on every block.  The
# wide attention kernel writes its QK products to VGPRs the same way (its
# 256-register accumulator is pinned to AGPRs by the asm P.V products).
EXTRA = {"sparse_attn_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "sparse_attn_wide.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    if src.endswith(".hip"):
        cmd = [_hipcc(), "-x", "hip", *DEVICE, *EXTRA.get(src, []), *COMMON, "-c", path, "-o", obj]
    else:
        cmd = [_hipcc(), *COMMON, "-D__HIP_PLATFORM_AMD__", "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libdsa.so; always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = HIP_SOURCES + CPP_SOURCES
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

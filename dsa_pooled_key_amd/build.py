"""Builds libdsa.so for gfx950 in-tree with hipcc.

Each source under csrc/ is compiled to an object with its own flags and the objects are linked
into dsa_pooled_key_amd/libdsa.so. Device code is compiled with packed-fp32 instructions
disabled; the host weight transforms with FMA contraction disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libdsa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

KERNELS = ["kpool_compress.hip", "cache_update.hip", "compact_pools.hip", "index_scores.hip",
           "topk_pools.hip",
           "expand_selection.hip", "sparse_mla_decode.hip", "masked_attn.hip", "measure.hip"]
HOST = ["dsa_api.cpp", "absorb.cpp"]

COMMON = ["-std=c++17", "-O3", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]
DEVICE = ["-x", "hip", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-ffp-contract=fast"]
HOST_ONLY = ["-ffp-contract=off"]
# Per-file additions. The MFMA-rate measurement keeps MFMA accumulators in the VGPR form (the
# form the production kernels get under their register pressure): in the accumulator-register
# form the compiler copies a 16x16 chain's result back every round, so the loop would measure
# those copies.
EXTRA = {"measure.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    flags = COMMON + (DEVICE if src.endswith(".hip") else HOST_ONLY) + EXTRA.get(src, [])
    cmd = [HIPCC] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    if res.stderr.strip() and verbose:
        print(res.stderr, file=sys.stderr)
    return obj


def build_library(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), KERNELS + HOST))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))

"""Builds libdsa.so for gfx950 in-tree with hipcc.

Each source under csrc/ is compiled to an object with its own flags and the objects are linked
into dsa_pooled_key_amd/libdsa.so. Device code is compiled with packed-fp32 instructions
disabled; the host weight transforms with FMA contraction disabled.

`python -m dsa_pooled_key_amd.build --trace` builds libdsa_trace.so beside it instead: the
same sources with DSA_PHASE_TRACE defined, so the decode-step kernels record per-block phase
timestamps (dsa_phase.hpp) for phase_trace.py. The product library never has them.
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


TRACE_LIB_PATH = os.path.join(HERE, "libdsa_trace.so")
TRACE_BUILD = os.path.join(ROOT, "_build_trace")


def _compile(src: str, verbose: bool, trace: bool = False) -> str:
    obj = os.path.join(TRACE_BUILD if trace else BUILD, os.path.basename(src) + ".o")
    flags = COMMON + (DEVICE if src.endswith(".hip") else HOST_ONLY) + EXTRA.get(src, [])
    if trace and src.endswith(".hip"):
        flags = flags + ["-DDSA_PHASE_TRACE"]
    cmd = [HIPCC] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    if res.stderr.strip() and verbose:
        print(res.stderr, file=sys.stderr)
    return obj


def build_library(verbose: bool = False, jobs: int = 8, trace: bool = False) -> str:
    """Compiles every source and links the library; returns its path (trace: the
    phase-timestamp library, libdsa_trace.so)."""
    out = TRACE_LIB_PATH if trace else LIB_PATH
    os.makedirs(TRACE_BUILD if trace else BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, trace), KERNELS + HOST))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv, trace="--trace" in sys.argv))

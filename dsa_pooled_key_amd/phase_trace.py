"""Per-block phase timeline of one decode step, from the trace library.

    python -m dsa_pooled_key_amd.build --trace        # once, on any machine with hipcc
    python -m dsa_pooled_key_amd.phase_trace [--workload fp8_mixed_b32] [--out FILE]

libdsa_trace.so is the product's sources built with DSA_PHASE_TRACE: thread 0 of every block
of the four decode-step kernels stores the 100 MHz constant clock at the points named in
PHASES (dsa_phase.hpp). This script runs the workload's step over enough input replicas to
leave its buffers out of the 256 MiB MALL (as bench.py does), clears the stamp tables, runs
one more step (launch by launch, not from a graph) and prints, per kernel and point, the
median, 10th and 90th percentile over the blocks of the time since the kernel's first block
started, in microseconds, plus the median per-block duration of each phase. Kernels start
after the previous one ends; the spans between them are not in the tables.
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

KERNELS = ("compact_index_scores", "topk_expand", "sparse_mla main", "sparse_mla combine")
# Per kernel: the points, in program order, that a block may stamp (slot: meaning).
PHASES = {
    0: {0: "block start", 1: "range known, query requested", 2: "query and flags landed",
        3: "keys landed, first tile scored", 4: "range scored"},
    1: {0: "block start", 1: "keys loaded, wave reductions", 2: "block reduction",
        3: "histogram scanned", 4: "cutoff key known", 5: "output positions known",
        6: "selection written", 7: "token-id tail written"},
    2: {0: "block start", 1: "token ids and rows resolved", 2: "prologue barrier (tile 0, query)",
        3: "first tile done", 4: "every tile done", 5: "teams merged", 6: "result stores issued"},
    3: {0: "block start", 1: "outputs stored"},
}
# The translation unit whose table holds each kernel's stamps.
TABLE_OF = {0: "scores", 1: "topk", 2: "mla", 3: "mla"}
N_KERNELS, N_BLOCKS, N_SLOTS = 4, 4096, 8
TICK_US = 0.01  # s_memrealtime runs at 100 MHz


def load_trace_library():
    from dsa_pooled_key_amd import binding, build
    if not os.path.exists(build.TRACE_LIB_PATH):
        raise SystemExit(f"{build.TRACE_LIB_PATH} is missing: run "
                         "`python -m dsa_pooled_key_amd.build --trace` first")
    binding.LIB_PATH = build.TRACE_LIB_PATH
    L = binding.lib()
    for name in set(TABLE_OF.values()):
        for fn in (f"dsa_phase_read_{name}", f"dsa_phase_clear_{name}"):
            f = getattr(L, fn)
            f.restype = ctypes.c_int
        getattr(L, f"dsa_phase_read_{name}").argtypes = [ctypes.c_void_p]
        getattr(L, f"dsa_phase_clear_{name}").argtypes = []
    return L


def read_tables(L):
    out = {}
    for name in set(TABLE_OF.values()):
        buf = np.zeros(N_KERNELS * N_BLOCKS * N_SLOTS, dtype=np.uint64)
        rc = getattr(L, f"dsa_phase_read_{name}")(buf.ctypes.data)
        if rc != 0:
            raise RuntimeError(f"dsa_phase_read_{name} returned {rc}")
        out[name] = buf.reshape(N_KERNELS, N_BLOCKS, N_SLOTS)
    return out


def summarise(tables):
    lines = []
    for k in range(N_KERNELS):
        t = tables[TABLE_OF[k]][k].astype(np.int64)
        started = t[:, 0] > 0
        if not started.any():
            continue
        t0 = t[started, 0].min()
        end = t[started].max()
        lines.append(f"### {KERNELS[k]}: {int(started.sum())} blocks, "
                     f"{(end - t0) * TICK_US:.2f} us from the first block's start to the last stamp")
        lines.append("")
        lines.append("| point | blocks | p10 us | median us | p90 us | median phase us |")
        lines.append("|---|---:|---:|---:|---:|---:|")
        prev = None
        for s, name in PHASES[k].items():
            have = started & (t[:, s] > 0)
            if not have.any():
                continue
            rel = (t[have, s] - t0) * TICK_US
            phase = ""
            if prev is not None:
                both = have & (t[:, prev] > 0)
                if both.any():
                    phase = f"{np.median((t[both, s] - t[both, prev]) * TICK_US):.2f}"
            lines.append(f"| {s} {name} | {int(have.sum())} | {np.percentile(rel, 10):.2f} | "
                         f"{np.median(rel):.2f} | {np.percentile(rel, 90):.2f} | {phase} |")
            prev = s
        lines.append("")
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="fp8_mixed_b32")
    ap.add_argument("--replicas", type=int, default=0,
                    help="input replicas rotated before the traced step (0: past 4x the MALL)")
    ap.add_argument("--out", default="", help="also write the summary to this file")
    args = ap.parse_args(argv)

    L = load_trace_library()
    import torch

    from dsa_pooled_key_amd import synth
    from dsa_pooled_key_amd.pipeline import DecodeStep, DeviceDecodeInputs

    dev = torch.device("cuda:0")
    di = synth.make_decode_inputs(args.workload)
    x0 = DeviceDecodeInputs.upload(di, dev)
    # Bytes one step touches, at most: score and flag rows, every pool's key, every selected
    # token's latent row. Enough replicas that four times the MALL passes between two uses.
    wl = di.wl
    key_row = x0.keys.shape[-1] * x0.keys.element_size() + (4 if x0.key_scales is not None else 0)
    kv_row = x0.kv.shape[-1] * x0.kv.element_size() + (4 if x0.kv_scales is not None else 0)
    touched = wl.Q * wl.pools * 5 + wl.B * wl.pools * key_row + wl.Q * wl.topk * kv_row
    reps = args.replicas or int(min(16, max(2, -(-4 * (256 << 20) // touched))))
    xs = [x0] + [DeviceDecodeInputs(**{k: (None if v is None else v.clone())
                                       for k, v in x0.__dict__.items()}) for _ in range(reps - 1)]
    steps = [DecodeStep(di.wl, x, di.scale, di.sm_scale) for x in xs]
    for st in steps[1:] + steps[1:]:  # warm the code paths, then push replica 0 out of the MALL
        st.run()
    torch.cuda.synchronize()
    for name in set(TABLE_OF.values()):
        rc = getattr(L, f"dsa_phase_clear_{name}")()
        if rc != 0:
            raise RuntimeError(f"dsa_phase_clear_{name} returned {rc}")
    steps[0].run()
    torch.cuda.synchronize()
    text = (f"## Phase timeline, {args.workload} ({reps} input replicas, one traced step "
            f"launched kernel by kernel)\n\n" + summarise(read_tables(L)))
    print(text, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text + "\n")


if __name__ == "__main__":
    sys.exit(main())

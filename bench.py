"""Decode throughput of the pooled-key DSA path on one MI355X.

One step = one pass of the decode chain over a batch: pool compaction with index scores (one
fused launch, dsa_compact_index_scores) -> top-k with token-id expansion (one fused launch,
dsa_topk_expand) -> sparse_mla_decode (every launch goes through the C ABI).
Default workload: 32 decode queries at contexts log-uniform in [4K, 131,072] tokens,
index_kpool 8, index_topk 4,096, fp8 pooled keys and fp8 paged 512-wide latent with per-row
scales, 32 indexer heads x 128 and 32 MLA heads.

Protocol: inputs are resident in HBM; R replicas of every per-step input (pooled keys and
scales, validity, q, w, q_abs, latent cache, block tables) are cycled step by step so the
distinct bytes touched exceed 1 GiB (four times the 256 MB Infinity Cache). Steps are
recorded into HIP graphs and replayed; HIP events bracket exactly K steps. Each stage is
also replayed alone (its own graph over the same replicas) and timed with events, which
gives the per-launch duration used for the roofline of the dominant kernel. The CPU oracle
is timed on a sample of the same batch.

Prints one JSON line (see the keys at the end of main()).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFS = 2500.0         # MI355X dense bf16 MFMA, TFLOP/s
MALL_BYTES = 256 << 20         # Infinity Cache
KERNEL_SOURCES = {
    "compact_index_scores": "index_scores.hip",
    "index_scores": "index_scores.hip",
    "sparse_mla_decode": "sparse_mla_decode.hip",
    "topk_expand": "topk_pools.hip",
    "compact_pools": "compact_pools.hip",
    "kpool_compress": "kpool_compress.hip",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


KERNEL_HEADERS = {
    "compact_index_scores": ("dsa_device.hpp", "dsa_score_range.hpp"),
    "index_scores": ("dsa_device.hpp", "dsa_score_range.hpp"),
    "topk_expand": ("dsa_device.hpp", "dsa_topk_row.hpp"),
}


def source_hash(kernel: str) -> str:
    path = os.path.join(ROOT, "dsa_pooled_key_amd", "csrc", KERNEL_SOURCES[kernel])
    h = hashlib.sha256(open(path, "rb").read())
    for dep in KERNEL_HEADERS.get(kernel, ("dsa_device.hpp",)):
        h.update(open(os.path.join(ROOT, "dsa_pooled_key_amd", "csrc", dep), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary of this kernel, if it was
    taken on the current source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------- algorithmic bytes

def algorithmic_bytes(di, n_valid, n_tokens):
    """Bytes the method must move per step, by stage (inputs once, outputs once)."""
    wl = di.wl
    Q, Hi, D, H, B, P, W = wl.Q, wl.index_heads, wl.index_dim, wl.heads, wl.B, wl.pools, wl.width
    key_row = D + 4 if wl.key_fp8 else 2 * D
    tok_row = 512 + 4 if wl.kv_fp8 else 2 * 512
    valid_pools = int(np.sum(n_valid[di.row_seq]))
    return {
        "compact_pools": B * P + B * P * 4 + B * 4,
        "index_scores": valid_pools * (key_row + 4) + Q * Hi * (2 * D + 4) + Q * P * 5,
        # flags of each row's sequence, candidate keys, q and w in; scores and cand out
        "compact_index_scores": Q * P + valid_pools * key_row + Q * Hi * (2 * D + 4) + Q * P * 5,
        "topk_expand": Q * P * 5 + Q * wl.kw * 4 + Q * W * 4,
        "sparse_mla_decode": n_tokens * tok_row + Q * W * 4 + Q * H * 512 * 2 + Q * H * (512 + 1) * 4,
        # the method's own bytes for the whole step (intermediates excluded)
        "step": valid_pools * key_row + B * P + Q * Hi * (2 * D + 4) + n_tokens * tok_row
                + Q * H * 512 * 2 + Q * H * 512 * 4 + Q * W * 4,
    }


# ---------------------------------------------------------------- GPU part

def cycle_percentiles(cycle_graph, reps, n_cycles, stream):
    """p10 / p50 / p90 of the per-step time over n_cycles replays of the replica cycle, each
    bracketed by its own HIP events on the replay stream."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_cycles)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        cycle_graph.replay()
        b.record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) / reps for a, b in ev])
    return {f"p{q}": round(float(np.percentile(t, q)), 5) for q in (10, 50, 90)}


def run_chain(name, steps, warmup, seed=0, replicas=0):
    """The whole chain on another workload: ms per step over HIP-graph replays of a cycle of
    input replicas (at least 1 GiB of distinct inputs), plus what the rooflines need."""
    import torch

    from dsa_pooled_key_amd import synth
    from dsa_pooled_key_amd.pipeline import DecodeStep, DeviceDecodeInputs

    dev = torch.device("cuda:0")
    t0 = time.time()
    di = synth.make_decode_inputs(name, seed=seed)
    wl = di.wl
    x0 = DeviceDecodeInputs.upload(di, dev)
    probe = DecodeStep(wl, x0, di.scale, di.sm_scale)
    probe.run()
    torch.cuda.synchronize()
    n_tokens = int((probe.token_ids >= 0).sum().item())
    n_cand = int(probe.cand.sum(dtype=torch.int64).item())
    n_valid = (di.pool_valid != 0).sum(axis=1)
    alg = algorithmic_bytes(di, n_valid, n_tokens)
    reps = replicas or int(min(16, max(2, -(-4 * MALL_BYTES // alg["step"]))))
    xs = [x0] + [DeviceDecodeInputs(**{k: (None if v is None else v.clone())
                                       for k, v in x0.__dict__.items()}) for _ in range(reps - 1)]
    stps = [probe] + [DecodeStep(wl, x, di.scale, di.sm_scale) for x in xs[1:]]
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    for i in range(max(warmup, reps)):
        stps[i % reps].run()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for st in stps:
            st.run()
    n_cycles = max(2, -(-steps // reps))
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(n_cycles):
        g.replay()
    b.record(stream)
    b.synchronize()
    ms = a.elapsed_time(b) / (n_cycles * reps)
    torch.cuda.set_stream(torch.cuda.default_stream())
    log(f"{name}: {ms * 1e3:.2f} us per step over {n_cycles * reps} steps, {reps} replicas "
        f"(inputs drawn and uploaded in {time.time() - t0:.1f}s)")
    out = {"di": di, "alg": alg, "ms": ms, "reps": reps, "steps": n_cycles * reps,
           "n_tokens": n_tokens, "n_cand": n_cand}
    del stps, xs, x0, probe, g
    torch.cuda.empty_cache()
    return out


def masked_check_line(args):
    """The dense masked-attention cross-check (topk_to_mask + mla_masked_attn) on the 32K
    decode workload's selection: microseconds per launch from graphs of several launches."""
    import torch

    from dsa_pooled_key_amd import binding as dsa
    from dsa_pooled_key_amd import synth
    from dsa_pooled_key_amd.pipeline import DecodeStep, DeviceDecodeInputs

    di = synth.make_decode_inputs("decode_b8_32k", seed=args.seed)
    wl = di.wl
    x = DeviceDecodeInputs.upload(di, torch.device("cuda:0"))
    st = DecodeStep(wl, x, di.scale, di.sm_scale)
    st.run()
    mask = dsa.topk_to_mask(st.token_ids, wl.S)
    out = torch.empty_like(st.out)
    lse = torch.empty_like(st.lse)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    fns = {"topk_to_mask": lambda: dsa.topk_to_mask(st.token_ids, wl.S, mask),
           "mla_masked_attn": lambda: dsa.mla_masked_attn(
               st.cfg, x.q_abs, mask, x.row_seq, x.kv, B=wl.B, sm_scale=di.sm_scale, out=out,
               lse=lse),
           "sparse_mla_decode": st.attend}
    res = {}
    for nm, fn in fns.items():
        fn()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(4):
                fn()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(5):
            g.replay()
        b.record(stream)
        b.synchronize()
        res[nm] = round(a.elapsed_time(b) / 20 * 1e3, 2)
    torch.cuda.set_stream(torch.cuda.default_stream())
    n_tok = int((st.token_ids >= 0).sum().item())
    return {"workload": f"{wl.name}: {wl.Q} rows, {wl.heads} heads, every masked token of an "
                        f"{wl.S}-position score row ({n_tok} tokens selected in all)",
            "launch_us": res}


def extra_lines(args):
    """X128 decode and C4 prefill, reported beside the main line."""
    extra = {}
    if not args.no_masked:
        extra["masked_check"] = masked_check_line(args)
    def decode_line(name, what):
        r = run_chain(name, args.extra_steps, args.warmup, args.seed)
        wl = r["di"].wl
        gbs = r["alg"]["step"] / (r["ms"] * 1e-3) / 1e9
        return {"workload": f"{wl.name}: {wl.Q} decode queries, {what}, kpool {wl.kpool}, "
                            f"topk {wl.topk}, bf16 keys and latent, "
                            f"{'paged 64-token blocks' if wl.paged else 'contiguous'}",
                "queries_per_s": round(wl.Q / (r["ms"] * 1e-3), 1), "ms_per_step": round(r["ms"], 5),
                "steps": r["steps"], "replicas": r["reps"],
                "algorithmic_bytes": r["alg"]["step"], "achieved_GBs": round(gbs, 1),
                "frac_of_peak_hbm": round(gbs / PEAK_HBM_GBS, 4)}

    if not args.no_x128:
        extra["x128"] = decode_line("decode_b8_128k", "every context 131072")
    if not args.no_decode_lines:
        extra["decode_b8_32k"] = decode_line("decode_b8_32k", "contexts uniform in [16384, 32768]")
        extra["decode_b4_256k"] = decode_line("decode_b4_256k", "every context 262144")
    if not args.no_prefill:
        r = run_chain("prefill_2048_64k", args.extra_steps, args.warmup, args.seed)
        wl = r["di"].wl
        flop = 2 * wl.index_heads * wl.index_dim * r["n_cand"] + 4 * wl.heads * 512 * r["n_tokens"]
        tfs = flop / (r["ms"] * 1e-3) / 1e12
        extra["prefill"] = {
            "workload": f"{wl.name}: {wl.Q} causal rows at positions {wl.S - wl.Q}..{wl.S - 1} of "
                        f"one {wl.S}-token sequence, kpool {wl.kpool}, topk {wl.topk}, bf16",
            "rows_per_s": round(wl.Q / (r["ms"] * 1e-3), 1), "ms_per_step": round(r["ms"], 5),
            "steps": r["steps"], "replicas": r["reps"],
            "flop": flop, "candidate_pools": r["n_cand"], "tokens_attended": r["n_tokens"],
            "roofline": {"bound": "mfma", "achieved": round(tfs, 2), "peak": PEAK_BF16_TFS,
                         "unit": "TFLOP/s", "frac": round(tfs / PEAK_BF16_TFS, 4)}}
        if not args.no_cpu_baseline:
            log("timing the CPU oracle on a prefill subsample")
            extra["prefill"]["cpu_baseline"] = run_cpu_baseline_rows(r["di"], args.prefill_cpu_rows,
                                                                     args.seed)
    return extra

def run_gpu(args):
    import torch

    from dsa_pooled_key_amd import binding as dsa
    from dsa_pooled_key_amd import synth
    from dsa_pooled_key_amd.pipeline import DecodeStep, DeviceDecodeInputs

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    t0 = time.time()
    di = synth.make_decode_inputs(args.workload, seed=args.seed)
    wl = di.wl
    log(f"inputs for {wl.name} drawn in {time.time() - t0:.1f}s; libdsa {dsa.version()}")
    x0 = DeviceDecodeInputs.upload(di, dev)
    probe = DecodeStep(wl, x0, di.scale, di.sm_scale)
    probe.run()
    torch.cuda.synchronize()
    n_valid = (di.pool_valid != 0).sum(axis=1)  # compact_pools' count per sequence
    n_tokens = int((probe.token_ids >= 0).sum().item())
    alg = algorithmic_bytes(di, n_valid, n_tokens)
    touched = alg["step"]
    reps = args.replicas or int(min(48, max(4, -(-4 * MALL_BYTES // touched))))
    log(f"step touches {touched / 2**20:.1f} MiB of algorithmic bytes; {reps} replicas "
        f"-> {reps * touched / 2**30:.2f} GiB distinct per cycle; {n_tokens} tokens attended")

    def clone(x):
        return DeviceDecodeInputs(**{k: (None if v is None else v.clone())
                                     for k, v in x.__dict__.items()})

    xs = [x0] + [clone(x0) for _ in range(reps - 1)]
    steps = [DecodeStep(wl, x, di.scale, di.sm_scale) for x in xs]
    for i in range(max(args.warmup, reps)):
        steps[i % reps].run()
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)

    def graph_of(fns):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for f in fns:
                f()
        return g

    g_cycle = graph_of([s.run for s in steps])
    g_single = [graph_of([s.run]) for s in steps]
    for i in range(args.warmup):
        g_single[i % reps].replay()
    torch.cuda.synchronize()

    def per_launch_us(fn, in_graph, replays):
        """One graph of in_graph launches of fn, replayed; microseconds per launch (the
        graph launch overhead spread over in_graph kernels)."""
        g = graph_of([fn] * in_graph)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(replays):
            g.replay()
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b) / (in_graph * replays) * 1e3

    def timed(cycle_graph, single_graphs, k):
        """Replay exactly k launches of the recorded work, rotating replicas; ms per one."""
        full, rest = divmod(k, len(single_graphs))
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(full):
            cycle_graph.replay()
        for i in range(rest):
            single_graphs[i].replay()
        stop.record(stream)
        stop.synchronize()
        return start.elapsed_time(stop) / k

    ms_step = timed(g_cycle, g_single, args.steps)
    log(f"decode step: {ms_step * 1e3:.2f} us ({wl.Q / ms_step * 1e3:.0f} queries/s)")
    pct = cycle_percentiles(g_cycle, reps, max(8, args.steps // reps), stream)

    # Per-stage durations: each stage alone, same replicas, same graph replay.
    stage_fns = {
        "compact_index_scores": lambda s: s.score(),
        "topk_expand": lambda s: s.topk(),
        "sparse_mla_decode": lambda s: s.attend(),
    }
    stage_us = {}
    for name, fn in stage_fns.items():
        gc = graph_of([(lambda s=s: fn(s)) for s in steps])
        gs = [graph_of([(lambda s=s: fn(s))]) for s in steps]
        for g in gs:
            g.replay()
        stage_us[name] = timed(gc, gs, args.steps) * 1e3
    log("stages (us): " + ", ".join(f"{k} {v:.2f}" for k, v in stage_us.items()))

    # Context build rate: kpool_compress over a token cache of the same shape (own inputs).
    ki = synth.make_kpool_inputs(args.workload, seed=args.seed, batch=args.kpool_batch)
    k = torch.from_numpy(ki.k.view(np.int16)).to(dev).view(torch.bfloat16)
    g_ = torch.from_numpy(ki.gate.view(np.int16)).to(dev).view(torch.bfloat16)
    ape = torch.from_numpy(ki.ape).to(dev)
    valid = torch.from_numpy(ki.valid).to(dev)
    kb, S = k.shape[0], k.shape[1]
    P = dsa.num_pools(S, wl.first_key, wl.kpool)
    pk = torch.empty((kb, P, wl.index_dim), dtype=torch.bfloat16, device=dev)
    pv = torch.empty((kb, P), dtype=torch.uint8, device=dev)
    cfg = steps[0].cfg
    kp_run = lambda: dsa.kpool_compress(cfg, k, g_, ape, valid, wl.first_key, pk, pv)  # noqa: E731
    kp_run()
    n_kp = max(5, args.steps // 40)
    kp_us = per_launch_us(kp_run, 4, n_kp)
    kp_tokens = kb * P * wl.kpool
    kp_bytes = kp_tokens * (wl.index_dim * 4 + 1) + kb * P * (wl.index_dim * 2 + 1)
    # fp8 writers: the same pooling stored as fp8 (codes + per-pool scale), and the latent
    # quantizer over a cache of 262,144 bf16 rows of 512 (two 131,072-token contexts).
    pk8 = torch.empty((kb, P, wl.index_dim), dtype=torch.uint8, device=dev)
    sc8 = torch.empty((kb, P), dtype=torch.float32, device=dev)
    kp8_run = lambda: dsa.kpool_compress_fp8(cfg, k, g_, ape, valid, wl.first_key, pk8, sc8, pv)  # noqa: E731
    kp8_run()
    kp8_us = per_launch_us(kp8_run, 4, n_kp)
    kp8_bytes = kp_tokens * (wl.index_dim * 4 + 1) + kb * P * (wl.index_dim + 4 + 1)
    n_lat = 262144
    lat = (torch.randn((n_lat, 512), device=dev) * 0.5).to(torch.bfloat16)
    lat_codes = torch.empty((n_lat, 512), dtype=torch.uint8, device=dev)
    lat_sc = torch.empty((n_lat,), dtype=torch.float32, device=dev)
    q_run = lambda: dsa.quantize_rows_fp8(lat, lat_codes, lat_sc)  # noqa: E731
    q_run()
    q_us = per_launch_us(q_run, 4, n_kp)
    q_bytes = n_lat * (512 * 2 + 512 + 4)
    del lat, lat_codes, lat_sc
    # Decode-time upkeep of the same token cache (one new token per sequence, each at a
    # position that completes a pool): k_norm of the staged key rows, indexer_store,
    # write_geom and pool_append (fp8 keys). Small latency-bound launches.
    f, kpl = wl.first_key, wl.kpool
    up_pos = torch.tensor([f + ((S - 1 - f) // kpl - 1 - 3 * i) * kpl + kpl - 1 for i in range(kb)],
                          dtype=torch.int32, device=dev)
    k_rows = k[:, 0].contiguous()
    g_rows = g_[:, 0].contiguous()
    ln_w = torch.ones((wl.index_dim,), dtype=torch.bfloat16, device=dev)
    ln_b = torch.zeros((wl.index_dim,), dtype=torch.bfloat16, device=dev)
    seq_len = up_pos + 1
    rs_, rp_ = torch.empty_like(up_pos), torch.empty_like(up_pos)
    ids_, nv_ = dsa.compact_pools(pv)
    upkeep = {
        "k_norm": lambda: dsa.k_norm(k_rows, ln_w, ln_b, 1e-5),
        "indexer_store": lambda: dsa.indexer_store(up_pos, k_rows, g_rows, k, g_, valid),
        "write_geom": lambda: dsa.write_geom(seq_len, rs_, rp_),
        "pool_append": lambda: dsa.pool_append(cfg, up_pos, k, g_, ape, valid, pk8, pv, ids_, nv_,
                                               first_key=f, pool_key_scales=sc8),
    }
    up_us = {}
    for nm, fn in upkeep.items():
        fn()
        up_us[nm] = per_launch_us(fn, 50, 10)
    torch.cuda.set_stream(torch.cuda.default_stream())

    return {
        "di": di, "alg": alg, "ms_step": ms_step, "pct": pct, "stage_us": stage_us, "reps": reps,
        "n_tokens": n_tokens, "kpool": {"us": kp_us, "tokens": kp_tokens, "bytes": kp_bytes,
                                        "batch": kb},
        "upkeep_us": up_us, "upkeep_batch": kb,
        "fp8_writers": {"kpool_us": kp8_us, "kpool_bytes": kp8_bytes, "quant_us": q_us,
                        "quant_rows": n_lat, "quant_bytes": q_bytes},
    }


# ---------------------------------------------------------------- CPU baseline

def run_cpu_baseline(di, sample_every: int, min_seconds: float = 10.0, max_passes: int = 8):
    """The oracle's whole decode chain on the host cores, over every `sample_every`-th query
    of one step, repeated until at least `min_seconds` have passed (at most `max_passes`)."""
    import oracle

    wl = di.wl
    rows = np.arange(0, wl.Q, sample_every)
    passes = 0
    t0 = time.perf_counter()
    while True:
        ids, nv = oracle.compact_pools(di.pool_valid)
        rs, rc = oracle.index_scores(di.q[rows], di.w[rows], di.row_seq[rows], di.row_pos[rows],
                                     di.keys, ids, nv, kpool=wl.kpool, first_key=wl.first_key,
                                     scale=di.scale, key_scales=di.key_scales)
        sel = oracle.topk_pools(rs, rc, wl.kw)
        tok = oracle.expand_selection(sel, di.row_seq[rows], di.row_pos[rows], di.valid,
                                      kpool=wl.kpool, index_topk=wl.topk,
                                      always_select_tail=wl.tail, first_key=wl.first_key)
        oracle.sparse_mla(di.q_abs[rows], tok, di.row_seq[rows], di.kv, sm_scale=di.sm_scale,
                          S=wl.S, kv_scales=di.kv_scales, block_table=di.block_table)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or passes >= max_passes:
            break
    return {"value": passes * len(rows) / dt, "unit": "queries/s", "cores": oracle.num_threads(),
            "host_cpu_count": os.cpu_count(), "kind": "oracle",
            "sample": f"{len(rows)} of the {wl.Q} queries of one step (every {sample_every}th), "
                      f"whole decode chain, {passes} passes, {dt:.1f} s wall"}


def run_cpu_baseline_rows(di, n_rows: int, seed: int, min_seconds: float = 10.0, max_passes: int = 16):
    """The oracle's whole chain on a seeded random subsample of n_rows query rows (prefill:
    rows of one sequence), repeated until min_seconds have passed; rows/s."""
    import oracle

    wl = di.wl
    rng = np.random.default_rng(seed + 4242)
    rows = np.sort(rng.choice(wl.Q, size=min(n_rows, wl.Q), replace=False))
    passes = 0
    t0 = time.perf_counter()
    while True:
        ids, nv = oracle.compact_pools(di.pool_valid)
        rs, rc = oracle.index_scores(di.q[rows], di.w[rows], di.row_seq[rows], di.row_pos[rows],
                                     di.keys, ids, nv, kpool=wl.kpool, first_key=wl.first_key,
                                     scale=di.scale, key_scales=di.key_scales)
        sel = oracle.topk_pools(rs, rc, wl.kw)
        tok = oracle.expand_selection(sel, di.row_seq[rows], di.row_pos[rows], di.valid,
                                      kpool=wl.kpool, index_topk=wl.topk,
                                      always_select_tail=wl.tail, first_key=wl.first_key)
        oracle.sparse_mla(di.q_abs[rows], tok, di.row_seq[rows], di.kv, sm_scale=di.sm_scale,
                          S=wl.S, kv_scales=di.kv_scales, block_table=di.block_table)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or passes >= max_passes:
            break
    return {"value": round(passes * len(rows) / dt, 2), "unit": "rows/s",
            "cores": oracle.num_threads(), "host_cpu_count": os.cpu_count(), "kind": "oracle",
            "sample": f"{len(rows)} of the {wl.Q} rows (seeded random subsample), whole chain, "
                      f"{passes} passes, {dt:.1f} s wall"}


def stream_read_line(replays: int = 10):
    """The achievable HBM read rate on this GPU: the library's streaming read of a 4 GiB
    buffer (16 times the Infinity Cache), HIP events around repeated launches."""
    import torch

    from dsa_pooled_key_amd import binding as dsa

    nbytes = 4 << 30
    buf = torch.ones((nbytes // 4,), dtype=torch.int32, device="cuda:0")
    sink = torch.zeros((1,), dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(2):
            dsa.stream_read(buf, sink)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(replays):
            dsa.stream_read(buf, sink)
        b.record(stream)
        b.synchronize()
    ms = a.elapsed_time(b) / replays
    gbs = nbytes / (ms * 1e-3) / 1e9
    del buf
    torch.cuda.empty_cache()
    log(f"streaming read: {gbs:.0f} GB/s over {nbytes >> 30} GiB")
    return {"GBs": round(gbs, 1), "bytes": nbytes, "launch_us": round(ms * 1e3, 1),
            "frac_of_nominal_peak": round(gbs / PEAK_HBM_GBS, 4)}


def mfma_rate_line(blocks: int = 1024, iters: int = 2048, launches: int = 5):
    """The matrix units' dense rate on this GPU for the MFMA shapes the kernels use: the
    library's MFMA loop (4 independent chains a wave, 4 waves a block, 4 blocks a CU), HIP
    events around repeated launches."""
    import torch

    from dsa_pooled_key_amd import binding as dsa

    out = torch.empty((blocks * 256,), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.Stream()
    res = {}
    with torch.cuda.stream(stream):
        for kind, (name, _) in dsa.MFMA_RATE_SHAPES.items():
            for _ in range(2):
                dsa.mfma_rate(kind, blocks, iters, out)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            flop = 0
            for _ in range(launches):
                flop += dsa.mfma_rate(kind, blocks, iters, out)
            b.record(stream)
            b.synchronize()
            tfs = flop / (a.elapsed_time(b) * 1e-3) / 1e12
            res[name] = round(tfs, 1)
            log(f"MFMA {name}: {tfs:.0f} TFLOP/s")
    return {"TFLOPs": res, "blocks": blocks, "waves_per_block": 4, "chains_per_wave": 4,
            "bf16_frac_of_nominal_peak": round(max(res[dsa.MFMA_RATE_SHAPES[0][0]],
                                                   res[dsa.MFMA_RATE_SHAPES[1][0]]) / PEAK_BF16_TFS, 4)}


def launch_gap_line(launches: int = 200, replays: int = 5):
    """The gap between dependent launches in a replayed graph: a graph of empty kernels on one
    stream (1 block, and 256 blocks), HIP events around the replays."""
    import torch

    from dsa_pooled_key_amd import binding as dsa

    stream = torch.cuda.Stream()
    res = {}
    for blocks in (1, 256):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(launches):
                dsa.empty_launch(blocks)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        with torch.cuda.stream(stream):
            for _ in range(replays):
                g.replay()
        b.record(stream)
        b.synchronize()
        res[f"{blocks}_block{'s' if blocks > 1 else ''}"] = round(a.elapsed_time(b) * 1e3 / (replays * launches), 3)
        del g
    log(f"graph launch gap: {res} us a launch")
    return {"us_per_launch": res, "launches_per_graph": launches}


# ---------------------------------------------------------------- main

def run_eager(args):
    """Profiling mode: the decode step launched eagerly (no graphs) over rotating replicas,
    optionally one stage only, so counter runs see plain dispatches."""
    import torch

    from dsa_pooled_key_amd import binding as dsa
    from dsa_pooled_key_amd import synth
    from dsa_pooled_key_amd.pipeline import DecodeStep, DeviceDecodeInputs

    di = synth.make_decode_inputs(args.workload, seed=args.seed)
    wl = di.wl
    x0 = DeviceDecodeInputs.upload(di, torch.device("cuda:0"))
    reps = args.replicas or 4
    xs = [x0] + [DeviceDecodeInputs(**{k: (None if v is None else v.clone())
                                       for k, v in x0.__dict__.items()}) for _ in range(reps - 1)]
    steps = [DecodeStep(wl, x, di.scale, di.sm_scale) for x in xs]
    for s in steps:
        s.run()
    torch.cuda.synchronize()
    fn = {"all": lambda s: s.run(), "select": lambda s: s.select(),
          "attend": lambda s: s.attend()}[args.eager]
    t0 = time.perf_counter()
    for i in range(args.steps):
        fn(steps[i % reps])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    print(json.dumps({"mode": f"eager:{args.eager}", "workload": wl.name, "steps": args.steps,
                      "replicas": reps, "wall_ms_per_step": dt / args.steps * 1e3,
                      "libdsa": dsa.version()}), flush=True)


def run_copy_calibration(args):
    """A plain device copy of a known size, for scaling the FETCH_SIZE / WRITE_SIZE
    counters: each launch reads and writes exactly `bytes`."""
    import torch

    n = args.copy_bytes
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "copy_calibration", "bytes_per_launch": n, "launches": args.steps}),
          flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="fp8_mixed_b32")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--replicas", type=int, default=0)
    ap.add_argument("--kpool-batch", type=int, default=8)
    ap.add_argument("--cpu-sample-every", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-x128", action="store_true", help="skip the X128 decode line")
    ap.add_argument("--no-prefill", action="store_true", help="skip the C4 prefill line")
    ap.add_argument("--no-decode-lines", action="store_true",
                    help="skip the decode_b8_32k and decode_b4_256k lines")
    ap.add_argument("--prefill-cpu-rows", type=int, default=128,
                    help="rows of the prefill workload in the oracle's timed subsample")
    ap.add_argument("--no-masked", action="store_true",
                    help="skip the dense masked-attention cross-check line")
    ap.add_argument("--extra-steps", type=int, default=60,
                    help="timed steps of the X128 and prefill lines")
    ap.add_argument("--eager", choices=["all", "select", "attend"], default=None,
                    help="profiling mode: eager launches only, no timing report")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="profiling mode: plain copies of --copy-bytes for counter scaling")
    ap.add_argument("--copy-bytes", type=int, default=256 << 20)
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        raise SystemExit(2)
    if args.copy_calibration:
        return run_copy_calibration(args)
    if args.eager:
        return run_eager(args)

    res = run_gpu(args)
    stream = stream_read_line()
    mfma = mfma_rate_line()
    gap = launch_gap_line()
    di, alg, ms = res["di"], res["alg"], res["ms_step"]
    wl = di.wl
    value = wl.Q / (ms * 1e-3)

    # Dominant kernel: the stage with the largest share of the step.
    dom = max(("compact_index_scores", "sparse_mla_decode", "topk_expand"),
              key=lambda k: res["stage_us"][k])
    dom_us = res["stage_us"][dom]
    achieved = alg[dom] / (dom_us * 1e-6) / 1e9
    traffic = measured_traffic(dom, wl.name)
    step_gbs = alg["step"] / (ms * 1e-3) / 1e9

    extra = extra_lines(args)
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        cpu = run_cpu_baseline(di, args.cpu_sample_every)

    kp = res["kpool"]
    line = {
        "metric": "DSA decode queries/s (index+topk+sparse MLA) at 128K ctx; % peak HBM GB/s",
        "value": round(value, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "ms_per_step_pct": res["pct"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8(e4m3)->bf16 mfma, f32 accumulate" if wl.kv_fp8 else "bf16 mfma, f32 accumulate",
        "data": "synthetic (seeded generators; no dataset or trained weights)",
        "config": {
            "workload": f"{wl.name}: {wl.Q} decode queries, contexts log-uniform in [4096, {wl.S}], "
                        f"kpool {wl.kpool}, topk {wl.topk}, indexer {wl.index_heads}x{wl.index_dim} "
                        f"{'fp8' if wl.key_fp8 else 'bf16'} keys, MLA {wl.heads} heads x 512 "
                        f"{'fp8' if wl.kv_fp8 else 'bf16'} latent, "
                        f"{'paged 64-token blocks' if wl.paged else 'contiguous'}",
            "global_batch": wl.Q,
            "seq_len": wl.S,
            "parallelism": "single GPU",
            "replicas": res["reps"],
            "tokens_attended_per_step": res["n_tokens"],
        },
        "roofline": {
            "bound": "hbm",
            "kernel": dom,
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "frac_of_measured_stream_read": round(achieved / stream["GBs"], 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": alg[dom],
            "launch_us": round(dom_us, 3),
        },
        "step_roofline": {
            "algorithmic_bytes": alg["step"],
            "achieved_GBs": round(step_gbs, 1),
            "frac_of_peak_hbm": round(step_gbs / PEAK_HBM_GBS, 4),
            "frac_of_measured_stream_read": round(step_gbs / stream["GBs"], 4),
        },
        "hbm_stream_read": stream,
        "mfma_measured": mfma,
        "graph_launch_gap": gap,
        "stage_us": {k: round(v, 3) for k, v in res["stage_us"].items()},
        "kpool_compress": {
            "tokens_per_s": round(kp["tokens"] / (kp["us"] * 1e-6), 1),
            "launch_us": round(kp["us"], 2),
            "achieved_GBs": round(kp["bytes"] / (kp["us"] * 1e-6) / 1e9, 1),
            "frac_of_peak_hbm": round(kp["bytes"] / (kp["us"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "sequences": kp["batch"],
        },
        "fp8_writers": {
            "kpool_compress_fp8": {
                "tokens_per_s": round(kp["tokens"] / (res["fp8_writers"]["kpool_us"] * 1e-6), 1),
                "launch_us": round(res["fp8_writers"]["kpool_us"], 2),
                "frac_of_peak_hbm": round(res["fp8_writers"]["kpool_bytes"]
                                          / (res["fp8_writers"]["kpool_us"] * 1e-6) / 1e9
                                          / PEAK_HBM_GBS, 4)},
            "quantize_rows_fp8": {
                "workload": f"{res['fp8_writers']['quant_rows']} latent rows of 512 bf16",
                "rows_per_s": round(res["fp8_writers"]["quant_rows"]
                                    / (res["fp8_writers"]["quant_us"] * 1e-6), 1),
                "launch_us": round(res["fp8_writers"]["quant_us"], 2),
                "frac_of_peak_hbm": round(res["fp8_writers"]["quant_bytes"]
                                          / (res["fp8_writers"]["quant_us"] * 1e-6) / 1e9
                                          / PEAK_HBM_GBS, 4)},
        },
        "decode_upkeep": {
            "workload": f"one new token in each of {res['upkeep_batch']} sequences of the "
                        f"{wl.name} token cache, each completing a pool (fp8 pooled keys)",
            "launch_us": {k_: round(v_, 2) for k_, v_ in res["upkeep_us"].items()},
        },
        "cpu_baseline": cpu,
    }
    if "prefill" in extra:
        pr = extra["prefill"]["roofline"]
        bf16 = max(v for k, v in mfma["TFLOPs"].items() if "bf16" in k)
        pr["frac_of_measured_mfma"] = round(pr["achieved"] / bf16, 4)
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

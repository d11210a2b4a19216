"""Seeded synthetic inputs for the pooled-key DSA decode path.

This module is the only code the GPU path and the CPU oracle share, and it holds none of the
method's arithmetic: it draws random numbers, encodes them (bf16 round-to-nearest-even,
saturating OCP e4m3 round-to-nearest-even with a per-row f32 scale), applies the
LayerNorm of the key recipe and lays the results out. It never pools, scores, selects or
attends. Everything is numpy on the host; arrays are bf16 bit patterns (``uint16``), e4m3
codes (``uint8``), ``float32``, ``int32`` and ``uint8`` masks.

Workloads (shapes from the model family the pages describe, GLM-5.3-Flash DSA: a
512-wide latent, at most 8 pool slots, an index_topk budget that is a multiple of the pool
size):

* ``tiny``            1 query, 1,024 token slots, kpool 4, topk 64, indexer 4x32, MLA 4 heads.
* ``decode_b8_32k``   8 queries, 32,768 slots, lengths U[16K, 32K], kpool 4, topk 2,048.
* ``decode_b4_256k``  4 queries at 262,144 tokens, paged bf16 latent in a shuffled block table.
* ``prefill_2048_64k`` 2,048 causal rows at positions 63,488..65,535 of a 65,536-token context.
* ``decode_b8_128k``  8 queries, every sequence at 131,072 tokens, otherwise decode_b8_32k.
* ``fp8_mixed_b32``   32 queries, log-uniform lengths in [4K, 131,072], kpool 8, topk 4,096,
  fp8 pooled keys and fp8 paged latent with per-row f32 scales, ~5% of slots invalid.
* ``fp8_mixed_b128``  fp8_mixed_b32's recipe with 128 queries (batch scaling).

Every workload also has an exact twin (``exact=True``): the same shapes with small dyadic
values (q, keys in multiples of 1/4 .. 1/32, w in multiples of 1/8, scale 2^-3, power-of-two
fp8 scales) for which every product and partial sum of the index score is exact in f32, so
pool and token selections must match bit for bit.

Each tensor has its own random stream: ``SeedSequence(seed).spawn`` in a fixed draw order.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

LATENT = 512
BLOCK = 64
_CHUNK = 1 << 22


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ----------------------------------------------------------------------------- encodings

def bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs: the
    largest finite pattern plus the rounding bias still fits in 32 bits)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    fi, fo = x.reshape(-1).view(np.uint32), out.reshape(-1)

    def run(i):
        u = fi[i:i + _CHUNK]
        fo[i:i + _CHUNK] = ((u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) >> 16).astype(np.uint16)

    idx = range(0, fi.size, _CHUNK)
    if len(idx) <= 1:
        for i in idx:
            run(i)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(run, idx))
    return out


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit pattern -> float32 (exact)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _e4m3_chunk(x: np.ndarray) -> np.ndarray:
    # Normal range: keep sign-less exponent + 3 mantissa bits of the binary32 pattern and
    # round the 20 dropped bits to nearest even; rebias 127 -> 7 (subtract 120 << 3).
    u = x.view(np.uint32)
    sign = ((u >> 24) & 0x80).astype(np.uint8)
    a = u & np.uint32(0x7FFFFFFF)
    keep = (a >> 20).astype(np.int32)
    rem = a & np.uint32(0xFFFFF)
    up = (rem > 0x80000) | ((rem == 0x80000) & ((keep & 1) == 1))
    code = np.clip(keep + up - 960, 0, 0x7E)
    # Below 2^-6 (binary32 pattern 0x3C800000) the grid is multiples of 2^-9.
    sub = a < np.uint32(0x3C800000)
    code[sub] = np.rint(np.abs(x[sub]) * np.float32(512.0)).astype(np.int32)
    return code.astype(np.uint8) | sign


def e4m3_codes(x) -> np.ndarray:
    """float -> OCP e4m3 ("FN") code: round to nearest, ties to even, saturating at +-448.
    Subnormals are multiples of 2^-9 below 2^-6."""
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    fi, fo = x.reshape(-1), out.reshape(-1)
    for i in range(0, fi.size, _CHUNK):
        fo[i:i + _CHUNK] = _e4m3_chunk(fi[i:i + _CHUNK])
    return out


def e4m3_quantize_rows(x, exact_pow2: bool = False):
    """Per-row scale s = amax/448 (1 for an all-zero row) and codes e4m3(x/s).
    With exact_pow2 the scale is the power of two 2^ceil(log2(amax/448)) instead, so that
    dyadic inputs stay exact. x is [..., n]; returns (codes uint8 [..., n], scales f32 [...])."""
    x = np.asarray(x, np.float32)
    amax = np.abs(x).max(axis=-1)
    s = (amax / np.float32(448.0)).astype(np.float32)
    if exact_pow2:
        s = np.exp2(np.ceil(np.log2(np.maximum(s, np.float32(1e-30))))).astype(np.float32)
    s = np.where(amax > 0, s, np.float32(1.0)).astype(np.float32)
    codes = np.empty(x.shape, np.uint8)
    xr, cr, sr = x.reshape(-1, x.shape[-1]), codes.reshape(-1, x.shape[-1]), s.reshape(-1)
    step = max(1, (1 << 22) // max(1, x.shape[-1]))

    def run(i):
        cr[i:i + step] = e4m3_codes(xr[i:i + step] / sr[i:i + step, None])

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(run, range(0, xr.shape[0], step)))
    return codes, s


def layer_norm_f32(x, eps: float = 1e-5) -> np.ndarray:
    """LayerNorm over the last axis with weight 1 and bias 0, in f32 (the key recipe)."""
    x = np.asarray(x, np.float32)
    mu = x.mean(axis=-1, keepdims=True, dtype=np.float32)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True, dtype=np.float32)
    return ((x - mu) / np.sqrt(var + np.float32(eps))).astype(np.float32)


# ----------------------------------------------------------------------------- workloads

@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int                 # sequences
    S: int                 # token slots per sequence
    Q: int                 # query rows
    kpool: int
    topk: int
    index_heads: int
    index_dim: int
    heads: int             # MLA heads
    first_key: int = 0
    tail: bool = False     # always_select_tail
    key_fp8: bool = False
    kv_fp8: bool = False
    paged: bool = False
    lengths: str = "full"  # full | minus3 | uniform_half | loguniform
    invalid_rate: float = 0.0   # extra invalid slots below the length
    rows: str = "decode"   # decode (one row per sequence at its last token) | prefill_tail
                           # (the last Q positions of sequence 0) | mixed (random sequences
                           # and positions, including positions before first_key)
    plain: bool = False    # un-normalised keys and U(0.5, 1.5) head weights (the tiny recipe)

    @property
    def pools(self) -> int:
        return (self.S - self.first_key) // self.kpool if self.S > self.first_key else 0

    @property
    def kw(self) -> int:
        return min(self.topk // self.kpool, self.pools)

    @property
    def width(self) -> int:
        return self.topk + (self.kpool - 1 if self.tail else 0)

    @property
    def max_blocks(self) -> int:
        return (self.S + BLOCK - 1) // BLOCK

    @property
    def prefill(self) -> bool:
        return self.rows != "decode"


WORKLOADS = {
    # The five measured workloads.
    "tiny": Workload("tiny", B=1, S=1024, Q=1, kpool=4, topk=64, index_heads=4, index_dim=32,
                     heads=4, lengths="minus3", plain=True),
    "decode_b8_32k": Workload("decode_b8_32k", B=8, S=32768, Q=8, kpool=4, topk=2048,
                              index_heads=32, index_dim=128, heads=32, lengths="uniform_half"),
    "decode_b4_256k": Workload("decode_b4_256k", B=4, S=262144, Q=4, kpool=4, topk=2048,
                               index_heads=32, index_dim=128, heads=32, paged=True),
    "prefill_2048_64k": Workload("prefill_2048_64k", B=1, S=65536, Q=2048, kpool=4, topk=2048,
                                 index_heads=32, index_dim=128, heads=32, rows="prefill_tail"),
    # Decode at a full 131,072-token context: decode_b8_32k's recipe with every sequence at
    # S (bench line "x128"; the same kernels and shapes as the parity-tested workloads).
    "decode_b8_128k": Workload("decode_b8_128k", B=8, S=131072, Q=8, kpool=4, topk=2048,
                               index_heads=32, index_dim=128, heads=32),
    "fp8_mixed_b32": Workload("fp8_mixed_b32", B=32, S=131072, Q=32, kpool=8, topk=4096,
                              index_heads=32, index_dim=128, heads=32, key_fp8=True,
                              kv_fp8=True, paged=True, lengths="loguniform", invalid_rate=0.05),
    # fp8_mixed_b32's recipe at 4x the batch (a batch-scaling line of the benchmark: the
    # same kernels with their fixed per-launch latency spread over more rows).
    "fp8_mixed_b128": Workload("fp8_mixed_b128", B=128, S=131072, Q=128, kpool=8, topk=4096,
                               index_heads=32, index_dim=128, heads=32, key_fp8=True,
                               kv_fp8=True, paged=True, lengths="loguniform", invalid_rate=0.05),
    # Small ragged workloads for parity at oracle-friendly sizes: sizes that are not multiples
    # of any tile, first_key > 0, tail slots, head counts below and above 32.
    "ragged_bf16": Workload("ragged_bf16", B=3, S=4999, Q=3, kpool=4, topk=200, index_heads=20,
                            index_dim=64, heads=40, first_key=3, tail=True,
                            lengths="uniform_half", invalid_rate=0.05),
    "ragged_fp8": Workload("ragged_fp8", B=5, S=3001, Q=5, kpool=8, topk=160, index_heads=32,
                           index_dim=128, heads=12, first_key=5, tail=True, key_fp8=True,
                           kv_fp8=True, paged=True, lengths="loguniform", invalid_rate=0.05),
    "ragged_prefill": Workload("ragged_prefill", B=2, S=2000, Q=70, kpool=2, topk=64,
                               index_heads=32, index_dim=32, heads=32, first_key=1,
                               lengths="uniform_half", rows="mixed"),
}

# Index score scale index_head_dim^-0.5 and MLA softmax scale qk_head_dim^-0.5 (qk_head_dim
# is 256 on GLM-5.3, so 1/16). The exact twins use 2^-3 for the index scale.
SM_SCALE = 1.0 / 16.0

# The "peaked" variant of a workload draws q_abs with this standard deviation instead of 0.5.
# A logit is SM_SCALE * sum_c q_c v_c over 512 channels with latent values of standard
# deviation 0.5, so its standard deviation is 16^-1 * sqrt(512) * 0.5 * std(q) = std(q)/sqrt(2);
# 3 * sqrt(2) gives logits of standard deviation 3, and a softmax over a few thousand tokens
# then puts most of its weight on a few dozen of them (at std 0.5 it is nearly uniform).
PEAKED_QABS_STD = 3.0 * math.sqrt(2.0)


def index_scale(wl: Workload, exact: bool) -> float:
    return 0.125 if exact else float(np.float32(wl.index_dim ** -0.5))


def _streams(seed: int, n: int):
    """n independent seed sequences, one per tensor, in a fixed order."""
    return np.random.SeedSequence(seed).spawn(n)


def _rng(ss) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(ss))


def _chunked(ss, shape, fill) -> np.ndarray:
    """A float32 array of `shape` filled in fixed 2^22-element chunks, chunk i from the i-th
    child stream of `ss`; chunks run on a thread pool, so the values do not depend on the
    number of threads."""
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    bounds = [(i, min(i + _CHUNK, n)) for i in range(0, n, _CHUNK)]
    kids = ss.spawn(len(bounds))

    def run(k):
        i0, i1 = bounds[k]
        fill(_rng(kids[k]), out[i0:i1])

    if len(bounds) == 1:
        run(0)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(run, range(len(bounds))))
    return out.reshape(shape)


def _normal(ss, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) float32."""
    def fill(g, o):
        g.standard_normal(out=o, dtype=np.float32)
        if std != 1.0:
            o *= np.float32(std)
    return _chunked(ss, shape, fill)


def _dyadic(ss, shape, denom: int, mmax: int) -> np.ndarray:
    """Uniform integers in [-mmax, mmax] divided by denom, as float32."""
    def fill(g, o):
        o[:] = g.integers(-mmax, mmax + 1, size=o.size).astype(np.float32) / np.float32(denom)
    return _chunked(ss, shape, fill)


def lengths(wl: Workload, rng) -> np.ndarray:
    """Valid length per sequence."""
    if wl.lengths == "minus3":
        return np.full(wl.B, wl.S - 3, np.int64)
    if wl.lengths == "uniform_half":
        return rng.integers(wl.S // 2, wl.S + 1, size=wl.B).astype(np.int64)
    if wl.lengths == "loguniform":
        lo = min(4096, max(1, wl.S // 32))
        u = rng.uniform(math.log(lo), math.log(wl.S), size=wl.B)
        return np.clip(np.rint(np.exp(u)), lo, wl.S).astype(np.int64)
    return np.full(wl.B, wl.S, np.int64)


def validity(wl: Workload, L: np.ndarray, rng):
    """Token validity [B,S] and pool validity [B,P] drawn together.

    With an invalid rate e, every slot below the length is invalid with probability e;
    this is sampled pool by pool: a pool wholly below the length is drawn all-valid with
    probability (1-e)^kpool, otherwise its slots are drawn from the distribution conditioned
    on at least one invalid slot. Without it, slots are valid exactly below the length.
    Pool validity is the drawn all-valid event, so it is not computed from the token mask."""
    B, S, KP, f, P = wl.B, wl.S, wl.kpool, wl.first_key, wl.pools
    e = wl.invalid_rate
    valid = np.zeros((B, S), np.uint8)
    pool_valid = np.zeros((B, P), np.uint8)
    for b in range(B):
        Lb = int(L[b])
        valid[b, :Lb] = 1
        whole = max(0, (Lb - f) // KP)
        if e > 0:
            ok = rng.random(whole) < (1.0 - e) ** KP
            pool_valid[b, :whole] = ok
            for p in np.nonzero(~ok)[0]:
                while True:
                    slot_ok = rng.random(KP) >= e
                    if not slot_ok.all():
                        break
                valid[b, f + p * KP: f + (p + 1) * KP] = slot_ok
            rest = np.r_[np.arange(0, min(f, Lb)), np.arange(f + whole * KP, Lb)]
            valid[b, rest] = rng.random(rest.size) >= e
        else:
            pool_valid[b, :whole] = 1
    return valid, pool_valid


def query_rows(wl: Workload, L: np.ndarray, rng):
    """(row_seq, row_pos) of the query rows."""
    Q = wl.Q
    if wl.rows == "prefill_tail":
        return np.zeros(Q, np.int32), (wl.S - Q + np.arange(Q)).astype(np.int32)
    if wl.rows == "mixed":
        seq = rng.integers(0, wl.B, Q).astype(np.int32)
        pos = np.array([rng.integers(0, L[b]) for b in seq], np.int32)
        pos[:2] = [0, max(0, wl.first_key - 1)]          # rows with no whole pool yet
        return seq, pos
    return np.arange(Q, dtype=np.int32), (L[:Q] - 1).astype(np.int32)


@dataclasses.dataclass
class DecodeInputs:
    """Inputs of the decode chain (compact_pools .. sparse MLA). Pooled keys are drawn here
    directly, as LayerNorm'd rows (the pooled cache is an input of this chain)."""
    wl: Workload
    exact: bool
    lengths: np.ndarray      # [B] int64
    valid: np.ndarray        # [B,S] u8 token validity (read by the tail of expand)
    pool_valid: np.ndarray   # [B,P] u8
    keys: np.ndarray         # [B,P,D] uint16 bf16 or uint8 e4m3
    key_scales: Optional[np.ndarray]   # [B,P] f32 (fp8 keys)
    q: np.ndarray            # [Q,Hi,D] uint16
    w: np.ndarray            # [Q,Hi] f32, index_heads^-0.5 already folded in
    row_seq: np.ndarray      # [Q] int32
    row_pos: np.ndarray      # [Q] int32
    q_abs: np.ndarray        # [Q,H,512] uint16
    kv: np.ndarray           # [rows,512] uint16 or uint8
    kv_scales: Optional[np.ndarray]    # [rows] f32 (fp8 latent)
    block_table: Optional[np.ndarray]  # [B,max_blocks] int32 (paged), -1 = unmapped
    scale: float
    sm_scale: float

    @property
    def kv_rows(self) -> int:
        return self.kv.shape[0]


def _layout_kv(wl: Workload, L: np.ndarray, rng_perm):
    """Rows of the latent cache and, for paged workloads, the block table: each sequence
    owns ceil(L_b / 64) blocks, all blocks shuffled across sequences; unmapped entries -1."""
    if not wl.paged:
        return wl.B * wl.S, None
    need = [int((int(l) + BLOCK - 1) // BLOCK) for l in L]
    total = int(sum(need))
    perm = rng_perm.permutation(total).astype(np.int32)
    table = np.full((wl.B, wl.max_blocks), -1, np.int32)
    o = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[o:o + n]
        o += n
    return total * BLOCK, table


def _q_abs(wl: Workload, ss, exact: bool, peaked: bool) -> np.ndarray:
    shape = (wl.Q, wl.heads, LATENT)
    if exact:
        return bf16_bits(_dyadic(ss, shape, 4, 4))
    return bf16_bits(_normal(ss, shape, PEAKED_QABS_STD if peaked else 0.5))


def peaked_q_abs(name: str, seed: int = 0) -> np.ndarray:
    """The q_abs of make_decode_inputs(name, seed, peaked=True), drawn alone."""
    return _q_abs(WORKLOADS[name], _streams(seed, 11)[6], False, True)


def make_decode_inputs(name: str, seed: int = 0, exact: bool = False,
                       peaked: bool = False) -> DecodeInputs:
    """The workload's decode inputs. ``peaked`` draws q_abs with PEAKED_QABS_STD (general
    inputs only); every other tensor is the same as without it."""
    wl = WORKLOADS[name]
    (s_len, s_valid, s_keys, s_kscale, s_q, s_w, s_qabs, s_kv, s_kvscale,
     s_perm, s_rows) = _streams(seed, 11)
    L = lengths(wl, _rng(s_len))
    valid, pool_valid = validity(wl, L, _rng(s_valid))
    B, P, D, Q, Hi, H = wl.B, wl.pools, wl.index_dim, wl.Q, wl.index_heads, wl.heads

    # pooled keys
    key_scales = None
    if exact:
        if wl.key_fp8:
            keys = e4m3_codes(_dyadic(s_keys, (B, P, D), 8, 8))
            key_scales = np.exp2(_rng(s_kscale).integers(-2, 2, size=(B, P))).astype(np.float32)
        else:
            keys = bf16_bits(_dyadic(s_keys, (B, P, D), 16, 16))
    else:
        kf = _normal(s_keys, (B, P, D))
        if not wl.plain:
            kf = layer_norm_f32(kf)
        if wl.key_fp8:
            keys, key_scales = e4m3_quantize_rows(kf)
        else:
            keys = bf16_bits(kf)

    # queries and head weights
    if exact:
        q = bf16_bits(_dyadic(s_q, (Q, Hi, D), 4, 4))
        w = _dyadic(s_w, (Q, Hi), 8, 12)
    else:
        q = bf16_bits(_normal(s_q, (Q, Hi, D)))
        if wl.plain:
            w = _rng(s_w).uniform(0.5, 1.5, size=(Q, Hi)).astype(np.float32)
        else:
            w = (_normal(s_w, (Q, Hi)) * np.float32(Hi ** -0.5)).astype(np.float32)

    row_seq, row_pos = query_rows(wl, L, _rng(s_rows))

    # latent side
    q_abs = _q_abs(wl, s_qabs, exact, peaked)
    rows, table = _layout_kv(wl, L, _rng(s_perm))
    kv_scales = None
    if wl.kv_fp8:
        if exact:
            kv = e4m3_codes(_dyadic(s_kv, (rows, LATENT), 8, 8))
            kv_scales = np.exp2(_rng(s_kvscale).integers(-2, 2, size=rows)).astype(np.float32)
        else:
            kv, kv_scales = e4m3_quantize_rows(_normal(s_kv, (rows, LATENT), 0.5))
    else:
        if exact:
            kv = bf16_bits(_dyadic(s_kv, (rows, LATENT), 4, 4))
        else:
            kv = bf16_bits(_normal(s_kv, (rows, LATENT), 0.5))
    return DecodeInputs(wl=wl, exact=exact, lengths=L, valid=valid, pool_valid=pool_valid,
                        keys=keys, key_scales=key_scales, q=q, w=w, row_seq=row_seq,
                        row_pos=row_pos, q_abs=q_abs, kv=kv, kv_scales=kv_scales,
                        block_table=table, scale=index_scale(wl, exact), sm_scale=SM_SCALE)


@dataclasses.dataclass
class KpoolInputs:
    """Inputs of kpool_compress: the per-token indexer cache."""
    wl: Workload
    exact: bool
    k: np.ndarray       # [B,S,D] uint16
    gate: np.ndarray    # [B,S,D] uint16
    ape: np.ndarray     # [KP,D] f32
    valid: np.ndarray   # [B,S] u8


def make_kpool_inputs(name: str, seed: int = 0, exact: bool = False,
                      batch: Optional[int] = None) -> KpoolInputs:
    """Token keys (LayerNorm'd N(0,1) rows; plain N(0,1) for ``tiny``), gate N(0,1), ape
    N(0,1) and the workload's validity (the same lengths and token mask as
    make_decode_inputs with the same seed). ``batch`` keeps only the first sequences.
    The exact twin has keys in multiples of 1/4, gate 0, and ape either 0 (uniform pool
    weights, kpool 4) or +-64 on one slot per channel (one-hot weights, kpool 8), so pooled
    keys are exact in bf16 and in e4m3; with fp8 pooled keys, channel 0 is +-7/4 on every
    token, which makes the per-row fp8 scale a power of two."""
    wl = WORKLOADS[name]
    s_len, s_valid = _streams(seed, 11)[:2]          # the decode inputs' lengths and masks
    (s_k, s_gate, s_ape, s_hot) = _streams(seed + 1000, 4)
    L = lengths(wl, _rng(s_len))
    valid, _ = validity(wl, L, _rng(s_valid))
    B = wl.B if batch is None else min(batch, wl.B)
    valid = np.ascontiguousarray(valid[:B])
    shape = (B, wl.S, wl.index_dim)
    if exact:
        kf = _dyadic(s_k, shape, 4, 4)
        if wl.key_fp8:
            # Channel 0 of every token key is +-7/4, so every one-hot pooled row has
            # amax 7/4 and the stored scale amax/448 is 2^-8; each value (a multiple of 1/4 of
            # magnitude at most 7/4) times 256 is then an e4m3 value, and the fp8 keys, their
            # scales and the scores computed from them are all exact.
            kf[..., 0] = np.where(kf[..., 0] < 0, np.float32(-1.75), np.float32(1.75))
        k = bf16_bits(kf)
        gate = np.zeros(shape, np.uint16)
        if wl.kpool == 8:
            hot = _rng(s_hot).integers(0, wl.kpool, size=wl.index_dim)
            ape = np.full((wl.kpool, wl.index_dim), -64.0, np.float32)
            ape[hot, np.arange(wl.index_dim)] = 64.0
        else:
            ape = np.zeros((wl.kpool, wl.index_dim), np.float32)
    else:
        kf = _normal(s_k, shape)
        k = bf16_bits(kf if wl.plain else layer_norm_f32(kf))
        gate = bf16_bits(_normal(s_gate, shape))
        ape = _normal(s_ape, (wl.kpool, wl.index_dim))
    return KpoolInputs(wl=wl, exact=exact, k=k, gate=gate, ape=ape, valid=valid)


def draw_token_ids(di: DecodeInputs, seed: int = 7, holes: float = 0.02) -> np.ndarray:
    """Synthetic attention sets for the sparse-MLA stage alone: per row, up to out_width
    distinct valid tokens at or before the row's position, ascending, a few slots replaced by
    -1, and -1 padding at the end (a row at a position with no valid token gets none).
    [Q, out_width] int32."""
    wl = di.wl
    rng = _rng(np.random.SeedSequence(seed))
    W = wl.width
    out = np.full((wl.Q, W), -1, np.int32)
    for r in range(wl.Q):
        b, pos = int(di.row_seq[r]), int(di.row_pos[r])
        pool = np.nonzero(di.valid[b, :pos + 1])[0]
        if pool.size == 0:
            continue
        n = int(min(W, pool.size) * rng.uniform(0.8, 1.0)) if r % 3 == 2 else min(W, pool.size)
        pick = np.sort(rng.choice(pool, size=n, replace=False)).astype(np.int32)
        pick[rng.random(n) < holes] = -1
        out[r, :n] = pick
    return out

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
* ``fp8_mixed_b32``   32 queries, log-uniform lengths in [4K, 131,072], kpool 8, topk 4,096,
  fp8 pooled keys and fp8 paged latent with per-row f32 scales, ~5% of slots invalid.

Every workload also has an exact twin (``exact=True``): the same shapes with small dyadic
values (q, keys in multiples of 1/4 .. 1/32, w in multiples of 1/8, scale 2^-3, power-of-two
fp8 scales) for which every product and partial sum of the index score is exact in f32, so
pool and token selections must match bit for bit.

Each tensor has its own random stream: ``SeedSequence(seed).spawn`` in a fixed draw order.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

LATENT = 512
BLOCK = 64


# ----------------------------------------------------------------------------- encodings

def bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = u + 0x7FFF + ((u >> 16) & 1)
    return ((rounded >> 16) & 0xFFFF).astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit pattern -> float32 (exact)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def e4m3_codes(x) -> np.ndarray:
    """float -> OCP e4m3 ("FN") code: round to nearest, ties to even, saturating at +-448.
    Subnormals are multiples of 2^-9 below 2^-6."""
    x = np.asarray(x, np.float32)
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.minimum(np.abs(x).astype(np.float64), 448.0)
    code = np.zeros(a.shape, np.uint8)
    sub = a < 2.0 ** -6
    code[sub] = np.rint(a[sub] * 512.0).astype(np.uint8)
    nrm = ~sub
    frac, ex = np.frexp(a[nrm])                 # a = frac * 2^ex, frac in [0.5, 1)
    mant = np.rint(frac * 16.0).astype(np.int64)  # 8..16, i.e. 1.mmm in eighths
    carry = mant == 16
    mant[carry] = 8
    ex = ex + carry
    biased = ex + 6                              # value = mant/8 * 2^(ex-1), bias 7
    code[nrm] = ((biased << 3) | (mant - 8)).astype(np.uint8)
    return code | sign


def e4m3_quantize_rows(x, exact_pow2: bool = False):
    """Per-row scale s = amax/448 (1 for an all-zero row) and codes e4m3(x/s).
    With exact_pow2 the scale is the power of two 2^ceil(log2(amax/448)) instead, so that
    dyadic inputs stay exact. x is [..., n]; returns (codes uint8 [..., n], scales f32 [...])."""
    x = np.asarray(x, np.float32)
    amax = np.abs(x).max(axis=-1)
    s = (amax / np.float32(448.0)).astype(np.float32)
    if exact_pow2:
        with np.errstate(divide="ignore"):
            s = np.where(amax > 0, np.exp2(np.ceil(np.log2(np.maximum(s, 1e-30)))), 1.0)
        s = s.astype(np.float32)
    s = np.where(amax > 0, s, np.float32(1.0)).astype(np.float32)
    codes = e4m3_codes(x / s[..., None])
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
    prefill: bool = False

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


WORKLOADS = {
    "tiny": Workload("tiny", B=1, S=1024, Q=1, kpool=4, topk=64, index_heads=4, index_dim=32,
                     heads=4),
    "decode_b8_32k": Workload("decode_b8_32k", B=8, S=32768, Q=8, kpool=4, topk=2048,
                              index_heads=32, index_dim=128, heads=32),
    "decode_b4_256k": Workload("decode_b4_256k", B=4, S=262144, Q=4, kpool=4, topk=2048,
                               index_heads=32, index_dim=128, heads=32, paged=True),
    "prefill_2048_64k": Workload("prefill_2048_64k", B=1, S=65536, Q=2048, kpool=4, topk=2048,
                                 index_heads=32, index_dim=128, heads=32, prefill=True),
    "fp8_mixed_b32": Workload("fp8_mixed_b32", B=32, S=131072, Q=32, kpool=8, topk=4096,
                              index_heads=32, index_dim=128, heads=32, key_fp8=True,
                              kv_fp8=True, paged=True),
}

# Index score scale index_head_dim^-0.5 and MLA softmax scale qk_head_dim^-0.5 (qk_head_dim
# is 256 on GLM-5.3, so 1/16). The exact twins use 2^-3 for the index scale.
SM_SCALE = 1.0 / 16.0


def index_scale(wl: Workload, exact: bool) -> float:
    return 0.125 if exact else float(np.float32(wl.index_dim ** -0.5))


def _streams(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def _dyadic(rng, shape, denom: int, mmax: int) -> np.ndarray:
    """Uniform integers in [-mmax, mmax] divided by denom, as float32."""
    return (rng.integers(-mmax, mmax + 1, size=shape) / float(denom)).astype(np.float32)


def lengths(wl: Workload, rng) -> np.ndarray:
    """Valid length per sequence."""
    if wl.name == "tiny":
        return np.array([wl.S - 3], np.int64)
    if wl.name == "decode_b8_32k":
        return rng.integers(wl.S // 2, wl.S + 1, size=wl.B).astype(np.int64)
    if wl.name == "fp8_mixed_b32":
        u = rng.uniform(math.log(4096), math.log(wl.S), size=wl.B)
        return np.clip(np.rint(np.exp(u)), 4096, wl.S).astype(np.int64)
    return np.full(wl.B, wl.S, np.int64)


def validity(wl: Workload, L: np.ndarray, rng):
    """Token validity [B,S] and pool validity [B,P] drawn together.

    For the mixed-length fp8 workload every slot below the length is invalid with
    probability 0.05; this is sampled pool by pool: a pool wholly below the length is drawn
    all-valid with probability 0.95^kpool, otherwise its slots are drawn from the
    distribution conditioned on at least one invalid slot. Elsewhere slots are valid exactly
    below the length. Pool validity is the drawn all-valid event, so it is not computed from
    the token mask here."""
    B, S, KP, f, P = wl.B, wl.S, wl.kpool, wl.first_key, wl.pools
    valid = np.zeros((B, S), np.uint8)
    pool_valid = np.zeros((B, P), np.uint8)
    for b in range(B):
        Lb = int(L[b])
        valid[b, :Lb] = 1
        whole = max(0, (Lb - f) // KP)
        if wl.name == "fp8_mixed_b32":
            p_ok = 0.95 ** KP
            ok = rng.random(whole) < p_ok
            pool_valid[b, :whole] = ok
            bad = np.nonzero(~ok)[0]
            for p in bad:
                while True:
                    slot_ok = rng.random(KP) >= 0.05
                    if not slot_ok.all():
                        break
                valid[b, f + p * KP: f + (p + 1) * KP] = slot_ok
            rest = np.arange(f + whole * KP, Lb)
            valid[b, rest] = rng.random(rest.size) >= 0.05
        else:
            pool_valid[b, :whole] = 1
    return valid, pool_valid


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
    """Rows of the latent cache and, for paged workloads, the block table."""
    if not wl.paged:
        return wl.B * wl.S, None
    if wl.name == "decode_b4_256k":
        nblk = wl.B * wl.max_blocks
        perm = rng_perm.permutation(nblk).astype(np.int32)
        return nblk * BLOCK, perm.reshape(wl.B, wl.max_blocks)
    need = [int((int(l) + BLOCK - 1) // BLOCK) for l in L]
    total = int(sum(need))
    perm = rng_perm.permutation(total).astype(np.int32)
    table = np.full((wl.B, wl.max_blocks), -1, np.int32)
    o = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[o:o + n]
        o += n
    return total * BLOCK, table


def make_decode_inputs(name: str, seed: int = 0, exact: bool = False) -> DecodeInputs:
    wl = WORKLOADS[name]
    (r_len, r_valid, r_keys, r_q, r_w, r_qabs, r_kv, r_perm) = _streams(seed, 8)
    L = lengths(wl, r_len)
    valid, pool_valid = validity(wl, L, r_valid)
    B, P, D, Q, Hi, H = wl.B, wl.pools, wl.index_dim, wl.Q, wl.index_heads, wl.heads

    # pooled keys
    key_scales = None
    if exact:
        if wl.key_fp8:
            kf = _dyadic(r_keys, (B, P, D), 8, 8)
            keys = e4m3_codes(kf)
            key_scales = np.exp2(r_keys.integers(-2, 2, size=(B, P))).astype(np.float32)
        else:
            keys = bf16_bits(_dyadic(r_keys, (B, P, D), 16, 16))
    else:
        kf = layer_norm_f32(r_keys.standard_normal((B, P, D), dtype=np.float32))
        if wl.key_fp8:
            keys, key_scales = e4m3_quantize_rows(kf)
        elif wl.name == "tiny":
            keys = bf16_bits(r_keys.standard_normal((B, P, D), dtype=np.float32))
        else:
            keys = bf16_bits(kf)

    # queries and head weights
    if exact:
        q = bf16_bits(_dyadic(r_q, (Q, Hi, D), 4, 4))
        w = _dyadic(r_w, (Q, Hi), 8, 12)
    else:
        q = bf16_bits(r_q.standard_normal((Q, Hi, D), dtype=np.float32))
        if wl.name == "tiny":
            w = r_w.uniform(0.5, 1.5, size=(Q, Hi)).astype(np.float32)
        else:
            w = (r_w.standard_normal((Q, Hi), dtype=np.float32) *
                 np.float32(Hi ** -0.5)).astype(np.float32)

    if wl.prefill:
        row_seq = np.zeros(Q, np.int32)
        row_pos = (wl.S - Q + np.arange(Q)).astype(np.int32)
    else:
        row_seq = np.arange(Q, dtype=np.int32)
        row_pos = (L - 1).astype(np.int32)

    # latent side
    if exact:
        q_abs = bf16_bits(_dyadic(r_qabs, (Q, H, LATENT), 4, 4))
    else:
        q_abs = bf16_bits(r_qabs.standard_normal((Q, H, LATENT), dtype=np.float32) * 0.5)
    rows, table = _layout_kv(wl, L, r_perm)
    kv_scales = None
    if wl.kv_fp8:
        if exact:
            kv = e4m3_codes(_dyadic(r_kv, (rows, LATENT), 8, 8))
            kv_scales = np.exp2(r_kv.integers(-2, 2, size=rows)).astype(np.float32)
        else:
            kv, kv_scales = e4m3_quantize_rows(
                r_kv.standard_normal((rows, LATENT), dtype=np.float32) * np.float32(0.5))
    else:
        if exact:
            kv = bf16_bits(_dyadic(r_kv, (rows, LATENT), 4, 4))
        else:
            kv = bf16_bits(r_kv.standard_normal((rows, LATENT), dtype=np.float32) * 0.5)
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
    N(0,1) and the workload's validity. ``batch`` keeps only the first sequences.
    The exact twin has keys in multiples of 1/4, gate 0, and ape either 0 (uniform pool
    weights, kpool 4) or +-64 on one slot per channel (one-hot weights, kpool 8), so pooled
    keys are exact in bf16 and in e4m3."""
    wl = WORKLOADS[name]
    (r_len, r_valid, r_k, r_gate, r_ape, r_hot) = _streams(seed + 1000, 6)
    L = lengths(wl, r_len)
    valid, _ = validity(wl, L, r_valid)
    B = wl.B if batch is None else min(batch, wl.B)
    valid = valid[:B]
    shape = (B, wl.S, wl.index_dim)
    if exact:
        k = bf16_bits(_dyadic(r_k, shape, 4, 4))
        gate = np.zeros(shape, np.uint16)
        if wl.kpool == 8:
            hot = r_hot.integers(0, wl.kpool, size=wl.index_dim)
            ape = np.full((wl.kpool, wl.index_dim), -64.0, np.float32)
            ape[hot, np.arange(wl.index_dim)] = 64.0
        else:
            ape = np.zeros((wl.kpool, wl.index_dim), np.float32)
    else:
        kf = r_k.standard_normal(shape, dtype=np.float32)
        k = bf16_bits(kf if wl.name == "tiny" else layer_norm_f32(kf))
        gate = bf16_bits(r_gate.standard_normal(shape, dtype=np.float32))
        ape = r_ape.standard_normal((wl.kpool, wl.index_dim), dtype=np.float32)
    return KpoolInputs(wl=wl, exact=exact, k=k, gate=gate, ape=ape, valid=valid)

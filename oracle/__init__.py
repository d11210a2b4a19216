"""CPU oracle for the pooled-key DSA path (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` import
this package. The GPU library and its Python binding never do, and the two share no code:
the oracle is the plain C file ``dsa_oracle.c`` (double-precision internals), wrapped here
with ctypes so that it takes and returns numpy arrays.

bf16 arrays are passed as ``uint16`` bit patterns and e4m3 arrays as ``uint8`` codes; every
other array has its natural numpy dtype. Each wrapper checks shapes and dtypes and returns
fresh output arrays.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB_PATH, build_oracle

__all__ = [
    "lib", "num_threads", "bf16_value", "e4m3_value", "bf16_from_float",
    "select_k", "out_width", "num_pools", "validate",
    "kpool_compress", "compact_pools", "index_scores", "topk_pools",
    "expand_selection", "sparse_mla", "absorb_q", "absorb_o",
]

_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_long
_D = ctypes.c_double


def lib():
    """Load (building first if needed) the oracle shared object."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build_oracle()
        L = ctypes.CDLL(LIB_PATH)
        L.orc_num_threads.restype = _I
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_bf16_value.restype = _D
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_value.restype = _D
        L.orc_bf16_from_float.argtypes = [ctypes.c_float]
        L.orc_bf16_from_float.restype = ctypes.c_uint16
        L.orc_select_k.argtypes = [_L, _L, _L]
        L.orc_select_k.restype = _L
        L.orc_out_width.argtypes = [_L, _L, _I]
        L.orc_out_width.restype = _L
        L.orc_num_pools.argtypes = [_L, _L, _L]
        L.orc_num_pools.restype = _L
        L.orc_validate.argtypes = [_L, _L, _L, _L]
        L.orc_validate.restype = _I
        L.orc_kpool_compress.argtypes = [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]
        L.orc_kpool_compress.restype = None
        L.orc_compact_pools.argtypes = [_I, _I, _P, _P, _P]
        L.orc_compact_pools.restype = None
        L.orc_index_scores.argtypes = [_I, _I, _I, _I, _I, _I, _I, _D, _P, _P, _P, _P, _P, _I,
                                       _P, _P, _P, _P, _P]
        L.orc_index_scores.restype = None
        L.orc_topk_pools.argtypes = [_I, _I, _I, _P, _P, _P]
        L.orc_topk_pools.restype = None
        L.orc_expand_selection.argtypes = [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P]
        L.orc_expand_selection.restype = None
        L.orc_sparse_mla.argtypes = [_I, _I, _I, _I, _D, _P, _P, _P, _P, _I, _P, _I, _P, _I, _I,
                                     _P, _P]
        L.orc_sparse_mla.restype = None
        L.orc_topk_to_mask.argtypes = [_I, _I, _I, _P, _P]
        L.orc_topk_to_mask.restype = None
        L.orc_masked_attn.argtypes = [_I, _I, _I, _I, _D, _P, _P, _P, _P, _I, _P, _P, _I, _I, _P,
                                      _P]
        L.orc_masked_attn.restype = None
        L.orc_layer_norm.argtypes = [_L, _I, _P, _P, _P, _D]
        L.orc_layer_norm.restype = None
        L.orc_indexer_store.argtypes = [_I, _I, _I, _P, _P, _P, _P, _P, _P]
        L.orc_indexer_store.restype = None
        L.orc_write_geom.argtypes = [_I, _P, _P, _P]
        L.orc_write_geom.restype = None
        L.orc_pool_append.argtypes = [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P]
        L.orc_pool_append.restype = None
        L.orc_e4m3_from_float.argtypes = [ctypes.c_float]
        L.orc_e4m3_from_float.restype = ctypes.c_uint8
        L.orc_quantize_rows.argtypes = [_L, _I, _P, _P, _P]
        L.orc_quantize_rows.restype = None
        L.orc_absorb_q.argtypes = [_I, _I, _I, _I, _I, _I, _P, _L, _P, _L, _P, ctypes.c_char_p, _I]
        L.orc_absorb_q.restype = _I
        L.orc_absorb_o.argtypes = [_I, _I, _I, _I, _I, _I, _P, _L, _P, _L, _P, ctypes.c_char_p, _I]
        L.orc_absorb_o.restype = _I
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _arr(a, dtype, shape=None, name="array"):
    a = np.ascontiguousarray(a)
    if a.dtype != np.dtype(dtype):
        raise TypeError(f"{name}: expected dtype {np.dtype(dtype)}, got {a.dtype}")
    if shape is not None and tuple(a.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(a.shape)}")
    return a


def num_threads() -> int:
    return int(lib().orc_num_threads())


def bf16_value(bits: int) -> float:
    return float(lib().orc_bf16_value(int(bits)))


def e4m3_value(code: int) -> float:
    return float(lib().orc_e4m3_value(int(code)))


def bf16_from_float(x: float) -> int:
    return int(lib().orc_bf16_from_float(float(x)))


def select_k(index_topk: int, index_kpool: int, n_pools: int) -> int:
    return int(lib().orc_select_k(index_topk, index_kpool, n_pools))


def out_width(index_topk: int, index_kpool: int, always_select_tail: bool) -> int:
    return int(lib().orc_out_width(index_topk, index_kpool, int(bool(always_select_tail))))


def num_pools(S: int, first_key: int, kpool: int) -> int:
    return int(lib().orc_num_pools(S, first_key, kpool))


def validate(index_kpool: int, index_topk: int, kv_lora_rank: int, local_heads: int) -> int:
    """0 = accepted, else the 1-based number of the first failing rule (see dsa_oracle.c)."""
    return int(lib().orc_validate(index_kpool, index_topk, kv_lora_rank, local_heads))


def kpool_compress(k, gate, ape, valid, kpool: int, first_key: int):
    """Returns (pool_keys [B,P,D] uint16 bf16 bits, pool_valid [B,P] uint8)."""
    k = _arr(k, np.uint16, name="k")
    B, S, D = k.shape
    gate = _arr(gate, np.uint16, (B, S, D), "gate")
    ape = _arr(ape, np.float32, (kpool, D), "ape")
    valid = _arr(valid, np.uint8, (B, S), "valid")
    if not 1 <= kpool <= 64:
        raise ValueError("kpool out of the oracle's range")
    P = num_pools(S, first_key, kpool)
    pk = np.zeros((B, P, D), np.uint16)
    pv = np.zeros((B, P), np.uint8)
    lib().orc_kpool_compress(B, S, D, kpool, first_key, _ptr(k), _ptr(gate), _ptr(ape),
                             _ptr(valid), _ptr(pk), _ptr(pv))
    return pk, pv


def e4m3_from_float(x: float) -> int:
    """OCP e4m3 code of a binary32 value: nearest, ties to even, saturating at +-448."""
    return int(lib().orc_e4m3_from_float(float(x)))


def quantize_rows(x):
    """Per-row fp8: x [..., n] float32 values -> (codes uint8 [..., n], scales f32 [...]) with
    s = amax/448 (1 for an all-zero row) and codes e4m3(x / s), both divisions in f32."""
    x = np.ascontiguousarray(x, np.float32)
    n = x.shape[-1]
    rows = x.size // n if n else 0
    codes = np.zeros(x.shape, np.uint8)
    scales = np.zeros(x.shape[:-1], np.float32)
    if rows:
        lib().orc_quantize_rows(rows, n, _ptr(x), _ptr(codes), _ptr(scales))
    return codes, scales


def kpool_compress_fp8(k, gate, ape, valid, kpool: int, first_key: int):
    """Pooled keys stored as fp8: the bf16 pooled key of kpool_compress, quantized per pool
    row by quantize_rows. Returns (codes [B,P,D] uint8, scales [B,P] f32, pool_valid [B,P])."""
    pk, pv = kpool_compress(k, gate, ape, valid, kpool, first_key)
    vals = (pk.astype(np.uint32) << 16).view(np.float32)
    codes, scales = quantize_rows(vals)
    return codes, scales, pv


def layer_norm(x, weight, bias, eps: float = 1e-5):
    """LayerNorm with a bias over the last axis of bf16 rows (k_norm): x [..., D] bf16 bits,
    weight/bias [D] bf16 bits -> new bf16 bits array (the input is not modified)."""
    x = np.array(x, np.uint16, copy=True, order="C")
    D = x.shape[-1]
    weight = _arr(weight, np.uint16, (D,), "weight")
    bias = _arr(bias, np.uint16, (D,), "bias")
    rows = x.size // D if D else 0
    if rows:
        lib().orc_layer_norm(rows, D, _ptr(x), _ptr(weight), _ptr(bias), float(eps))
    return x


def indexer_store(pos, k_row, gate_row, k_cache, gate_cache, valid):
    """Returns updated copies (k_cache, gate_cache, valid) after storing each sequence's staged
    row at pos[b] (when 0 <= pos[b] < S) and marking it valid."""
    k_cache = np.array(k_cache, np.uint16, copy=True, order="C")
    B, S, D = k_cache.shape
    gate_cache = np.array(gate_cache, np.uint16, copy=True, order="C").reshape(B, S, D)
    valid = np.array(valid, np.uint8, copy=True, order="C").reshape(B, S)
    pos = _arr(pos, np.int32, (B,), "pos")
    k_row = _arr(k_row, np.uint16, (B, D), "k_row")
    gate_row = _arr(gate_row, np.uint16, (B, D), "gate_row")
    lib().orc_indexer_store(B, S, D, _ptr(pos), _ptr(k_row), _ptr(gate_row), _ptr(k_cache),
                            _ptr(gate_cache), _ptr(valid))
    return k_cache, gate_cache, valid


def write_geom(seq_len):
    """Decode geometry from the live lengths: (row_seq [B], row_pos [B]) int32."""
    seq_len = _arr(seq_len, np.int32, name="seq_len")
    B = seq_len.shape[0]
    rs = np.zeros(B, np.int32)
    rp = np.zeros(B, np.int32)
    lib().orc_write_geom(B, _ptr(seq_len), _ptr(rs), _ptr(rp))
    return rs, rp


def pool_append(pos, k, gate, ape, valid, pool_keys, pool_valid, ids, n_valid, *, kpool: int,
                first_key: int):
    """The pool each sequence's new token (at pos[b]) completes: its key and validity as
    kpool_compress computes them, and, when valid, its id appended to the compacted list.
    Returns updated copies (pool_keys, pool_valid, ids, n_valid)."""
    k = _arr(k, np.uint16, name="k")
    B, S, D = k.shape
    gate = _arr(gate, np.uint16, (B, S, D), "gate")
    ape = _arr(ape, np.float32, (kpool, D), "ape")
    valid = _arr(valid, np.uint8, (B, S), "valid")
    P = num_pools(S, first_key, kpool)
    pos = _arr(pos, np.int32, (B,), "pos")
    pk = np.array(pool_keys, np.uint16, copy=True, order="C").reshape(B, P, D)
    pv = np.array(pool_valid, np.uint8, copy=True, order="C").reshape(B, P)
    ids = np.array(ids, np.int32, copy=True, order="C").reshape(B, P)
    nv = np.array(n_valid, np.int32, copy=True, order="C").reshape(B)
    lib().orc_pool_append(B, S, D, kpool, first_key, _ptr(pos), _ptr(k), _ptr(gate), _ptr(ape),
                          _ptr(valid), _ptr(pk), _ptr(pv), _ptr(ids), _ptr(nv))
    return pk, pv, ids, nv


def compact_pools(pool_valid):
    """Returns (ids [B,P] int32, n_valid [B] int32)."""
    pv = _arr(pool_valid, np.uint8, name="pool_valid")
    B, P = pv.shape
    ids = np.zeros((B, P), np.int32)
    nv = np.zeros((B,), np.int32)
    lib().orc_compact_pools(B, P, _ptr(pv), _ptr(ids), _ptr(nv))
    return ids, nv


def index_scores(q, w, row_seq, row_pos, keys, ids, n_valid, *, kpool: int, first_key: int,
                 scale: float, key_scales=None):
    """q [Q,Hi,D] bf16 bits; keys [B,P,D] bf16 bits (uint16) or e4m3 codes (uint8, then
    key_scales [B,P] f32). Returns (scores [Q,P] f32, cand [Q,P] uint8)."""
    q = _arr(q, np.uint16, name="q")
    Q, Hi, D = q.shape
    w = _arr(w, np.float32, (Q, Hi), "w")
    row_seq = _arr(row_seq, np.int32, (Q,), "row_seq")
    row_pos = _arr(row_pos, np.int32, (Q,), "row_pos")
    keys = np.ascontiguousarray(keys)
    fp8 = keys.dtype == np.uint8
    if not fp8:
        keys = _arr(keys, np.uint16, name="keys")
    B, P, Dk = keys.shape
    if Dk != D:
        raise ValueError("key width differs from query width")
    if fp8:
        key_scales = _arr(key_scales, np.float32, (B, P), "key_scales")
    ids = _arr(ids, np.int32, (B, P), "ids")
    n_valid = _arr(n_valid, np.int32, (B,), "n_valid")
    if Q and (row_seq.min() < 0 or row_seq.max() >= B):
        raise ValueError("row_seq out of range")
    scores = np.zeros((Q, P), np.float32)
    cand = np.zeros((Q, P), np.uint8)
    lib().orc_index_scores(Q, B, P, Hi, D, kpool, first_key, float(scale), _ptr(q), _ptr(w),
                           _ptr(row_seq), _ptr(row_pos), _ptr(keys), int(fp8),
                           _ptr(key_scales) if fp8 else None, _ptr(ids), _ptr(n_valid),
                           _ptr(scores), _ptr(cand))
    return scores, cand


def topk_pools(scores, cand, kw: int):
    """Returns sel [Q,kw] int32, ascending pool ids padded with -1."""
    scores = _arr(scores, np.float32, name="scores")
    Q, P = scores.shape
    cand = _arr(cand, np.uint8, (Q, P), "cand")
    sel = np.zeros((Q, kw), np.int32)
    lib().orc_topk_pools(Q, P, kw, _ptr(scores), _ptr(cand), _ptr(sel))
    return sel


def expand_selection(sel, row_seq, row_pos, valid, *, kpool: int, index_topk: int,
                     always_select_tail: bool, first_key: int):
    """Returns token_ids [Q, out_width] int32."""
    sel = _arr(sel, np.int32, name="sel")
    Q, kw = sel.shape
    if kw * kpool > index_topk:
        raise ValueError("selection wider than the index_topk budget")
    row_seq = _arr(row_seq, np.int32, (Q,), "row_seq")
    row_pos = _arr(row_pos, np.int32, (Q,), "row_pos")
    valid = _arr(valid, np.uint8, name="valid")
    B, S = valid.shape
    W = out_width(index_topk, kpool, always_select_tail)
    out = np.zeros((Q, W), np.int32)
    lib().orc_expand_selection(Q, kw, kpool, index_topk, int(bool(always_select_tail)), S,
                               first_key, _ptr(sel), _ptr(row_seq), _ptr(row_pos), _ptr(valid),
                               _ptr(out))
    return out


def sparse_mla(q_abs, token_ids, row_seq, kv, *, sm_scale: float, S: int = 0, kv_scales=None,
               block_table=None, block_size: int = 64):
    """q_abs [Q,H,C] bf16 bits; token_ids [Q,W]; kv [rows,C] bf16 bits or e4m3 codes
    (then kv_scales [rows] f32). Contiguous when block_table is None (row = b*S + t), else
    paged with block_table [B, max_blocks]. Returns (out [Q,H,C] f32, lse [Q,H] f32)."""
    q_abs = _arr(q_abs, np.uint16, name="q_abs")
    Q, H, C = q_abs.shape
    token_ids = _arr(token_ids, np.int32, name="token_ids")
    if token_ids.shape[0] != Q:
        raise ValueError("token_ids rows differ from q_abs rows")
    W = token_ids.shape[1]
    row_seq = _arr(row_seq, np.int32, (Q,), "row_seq")
    kv = np.ascontiguousarray(kv)
    fp8 = kv.dtype == np.uint8
    if not fp8:
        kv = _arr(kv, np.uint16, name="kv")
    kv = kv.reshape(-1, C)
    rows = kv.shape[0]
    if fp8:
        kv_scales = _arr(kv_scales, np.float32, name="kv_scales").reshape(-1)
        if kv_scales.shape[0] != rows:
            raise ValueError("kv_scales must hold one scale per latent row")
    max_blocks = 0
    if block_table is not None:
        block_table = _arr(block_table, np.int32, name="block_table")
        max_blocks = block_table.shape[1]
    # The oracle trusts its inputs, so check every address before calling it.
    for r in range(Q):
        b = int(row_seq[r])
        t = token_ids[r][token_ids[r] >= 0].astype(np.int64)
        if t.size == 0:
            continue
        if block_table is not None:
            blk = block_table[b][t // block_size].astype(np.int64)
            phys = blk * block_size + t % block_size
        else:
            phys = b * S + t
        if phys.min() < 0 or phys.max() >= rows:
            raise ValueError(f"row {r}: latent address out of range")
    out = np.zeros((Q, H, C), np.float32)
    lse = np.zeros((Q, H), np.float32)
    lib().orc_sparse_mla(Q, H, C, W, float(sm_scale), _ptr(q_abs), _ptr(token_ids),
                         _ptr(row_seq), _ptr(kv), int(fp8), _ptr(kv_scales) if fp8 else None,
                         int(S), _ptr(block_table), max_blocks, block_size, _ptr(out), _ptr(lse))
    return out, lse


def topk_to_mask(token_ids, S: int):
    """[Q, W] token ids -> [Q, S] u8 mask of the tokens present."""
    token_ids = _arr(token_ids, np.int32, name="token_ids")
    Q, W = token_ids.shape
    mask = np.zeros((Q, S), np.uint8)
    lib().orc_topk_to_mask(Q, W, S, _ptr(token_ids), _ptr(mask))
    return mask


def masked_attn(q_abs, mask, row_seq, kv, *, sm_scale: float, kv_scales=None, block_table=None,
                block_size: int = 64):
    """Dense attention over every masked token of each row: q_abs [Q,H,C] bf16 bits; mask
    [Q,S] u8; kv as sparse_mla (contiguous rows b*S + t, or paged). Returns (out, lse)."""
    q_abs = _arr(q_abs, np.uint16, name="q_abs")
    Q, H, C = q_abs.shape
    mask = _arr(mask, np.uint8, name="mask")
    S = mask.shape[1]
    row_seq = _arr(row_seq, np.int32, (Q,), "row_seq")
    kv = np.ascontiguousarray(kv)
    fp8 = kv.dtype == np.uint8
    if not fp8:
        kv = _arr(kv, np.uint16, name="kv")
    kv = kv.reshape(-1, C)
    rows = kv.shape[0]
    if fp8:
        kv_scales = _arr(kv_scales, np.float32, name="kv_scales").reshape(-1)
    max_blocks = 0
    if block_table is not None:
        block_table = _arr(block_table, np.int32, name="block_table")
        max_blocks = block_table.shape[1]
    for r in range(Q):  # the oracle trusts its inputs: check every address first
        t = np.nonzero(mask[r])[0]
        if t.size == 0:
            continue
        b = int(row_seq[r])
        if block_table is not None:
            blk = t // block_size
            ok = blk < max_blocks
            ent = np.where(ok, block_table[b][np.minimum(blk, max_blocks - 1)], -1)
            phys = np.where(ent >= 0, ent.astype(np.int64) * block_size + t % block_size, 0)
        else:
            phys = b * S + t
        if phys.max() >= rows:
            raise ValueError(f"row {r}: latent address out of range")
    out = np.zeros((Q, H, C), np.float32)
    lse = np.zeros((Q, H), np.float32)
    lib().orc_masked_attn(Q, H, C, S, float(sm_scale), _ptr(q_abs), _ptr(mask), _ptr(row_seq),
                          _ptr(kv), int(fp8), _ptr(kv_scales) if fp8 else None,
                          _ptr(block_table), max_blocks, block_size, _ptr(out), _ptr(lse))
    return out, lse


class OracleRefusal(ValueError):
    def __init__(self, code, msg):
        super().__init__(msg)
        self.code = code


def absorb_q(q_b, kv_b, *, heads, nope, rope, vd, kvl, ql):
    """Returns q_absorb [heads*kvl, ql] f32, or raises OracleRefusal."""
    q_b = _arr(q_b, np.float32, name="q_b").reshape(-1)
    kv_b = _arr(kv_b, np.float32, name="kv_b").reshape(-1)
    ok = rope == 0 and q_b.size == heads * (nope + rope) * ql and \
        kv_b.size == heads * (nope + vd) * kvl
    # On a refusal the C side returns before writing, so a 1-element buffer is enough.
    out = np.zeros((heads * kvl, ql) if ok else (1,), np.float32)
    msg = ctypes.create_string_buffer(256)
    rc = lib().orc_absorb_q(heads, nope, rope, vd, kvl, ql, _ptr(q_b), q_b.size, _ptr(kv_b),
                            kv_b.size, _ptr(out), msg, 256)
    if rc != 0:
        raise OracleRefusal(rc, msg.value.decode())
    return out


def absorb_o(o_local, kv_b_local, *, heads, nope, rope, vd, kvl, hidden):
    """Returns o_absorb [hidden, heads*kvl] f32, or raises OracleRefusal."""
    o_local = _arr(o_local, np.float32, name="o_local").reshape(-1)
    kv_b_local = _arr(kv_b_local, np.float32, name="kv_b_local").reshape(-1)
    ok = rope == 0 and o_local.size == hidden * heads * vd and \
        kv_b_local.size == heads * (nope + vd) * kvl
    out = np.zeros((hidden, heads * kvl), np.float32) if ok else np.zeros(1, np.float32)
    msg = ctypes.create_string_buffer(256)
    rc = lib().orc_absorb_o(heads, nope, rope, vd, kvl, hidden, _ptr(o_local), o_local.size,
                            _ptr(kv_b_local), kv_b_local.size, _ptr(out), msg, 256)
    if rc != 0:
        raise OracleRefusal(rc, msg.value.decode())
    return out

"""ctypes binding of libdsa (include/dsa.h): argument marshalling only.

Every function here checks tensor devices, dtypes, shapes and contiguity, allocates outputs
that were not passed in (plain torch allocations on the input's device), and calls the C
entry point of the same name on the current torch stream. All arithmetic happens in the HIP
kernels; there is no fallback path. Loading fails loudly when libdsa.so has not been built.

Tensor conventions: bf16 data is ``torch.bfloat16``; fp8 data is OCP e4m3 passed as
``torch.float8_e4m3fn`` or as its raw ``torch.uint8`` codes; ids are ``torch.int32``; masks
are ``torch.uint8``.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsa.so")

DSA_BF16, DSA_F32, DSA_FP8_E4M3 = 0, 1, 2
ERROR_NAMES = {
    -1: "DSA_ERR_NULL_ARG", -2: "DSA_ERR_BAD_SIZE", -3: "DSA_ERR_BAD_DTYPE",
    -4: "DSA_ERR_KPOOL_OR_TOPK_ZERO", -5: "DSA_ERR_TOPK_NOT_MULTIPLE", -6: "DSA_ERR_KPOOL_GT_MAX",
    -7: "DSA_ERR_KV_LORA_ZERO", -8: "DSA_ERR_KV_LORA_NOT_512", -9: "DSA_ERR_ZERO_HEADS",
    -10: "DSA_ERR_ROPE_UNSUPPORTED", -11: "DSA_ERR_ELEM_COUNT", -12: "DSA_ERR_WORKSPACE",
    -13: "DSA_ERR_HIP", -14: "DSA_ERR_UNSUPPORTED",
}
EXPORTED = [
    "dsa_last_error", "dsa_version", "dsa_config_validate", "dsa_select_k", "dsa_out_width",
    "dsa_num_pools", "dsa_kpool_compress", "dsa_kpool_compress_fp8", "dsa_quantize_rows_fp8",
    "dsa_k_norm", "dsa_indexer_store", "dsa_write_geom", "dsa_pool_append",
    "dsa_topk_to_mask", "dsa_mla_masked_attn",
    "dsa_compact_pools", "dsa_index_scores",
    "dsa_compact_index_scores",
    "dsa_topk_workspace", "dsa_topk_pools_workspace", "dsa_topk_pools", "dsa_expand_selection", "dsa_topk_expand",
    "dsa_sparse_mla_decode_workspace",
    "dsa_sparse_mla_decode", "dsa_sparse_mla_decode_noalloc", "dsa_stream_read", "dsa_empty_launch", "dsa_mfma_rate", "dsa_absorb_q", "dsa_absorb_o", "dsa_f32_to_bf16_rne",
]


class DsaError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {message}")
        self.code = code


class Config(ctypes.Structure):
    """dsa_config: per-layer geometry (mod.rs, Glm5NextDsaConfig)."""
    _fields_ = [(n, ctypes.c_int32) for n in (
        "index_heads", "index_head_dim", "index_kpool", "index_topk", "always_select_tail",
        "heads", "kv_lora_rank", "qk_nope_head_dim", "qk_rope_head_dim", "v_head_dim",
        "q_lora_rank", "hidden")]

    @classmethod
    def make(cls, *, index_heads, index_head_dim, index_kpool, index_topk, heads,
             always_select_tail=False, kv_lora_rank=512, qk_nope_head_dim=256,
             qk_rope_head_dim=0, v_head_dim=256, q_lora_rank=0, hidden=0):
        return cls(index_heads, index_head_dim, index_kpool, index_topk, int(always_select_tail),
                   heads, kv_lora_rank, qk_nope_head_dim, qk_rope_head_dim, v_head_dim,
                   q_lora_rank, hidden)


_lib = None
_P, _I, _I64, _SZ, _F = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t,
                         ctypes.c_float)
_CFG = ctypes.POINTER(Config)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "dsa_last_error": ([], ctypes.c_char_p),
            "dsa_version": ([], ctypes.c_char_p),
            "dsa_config_validate": ([_CFG], _I),
            "dsa_select_k": ([_CFG, _I64], _I64),
            "dsa_out_width": ([_CFG], _I64),
            "dsa_num_pools": ([_I64, _I64, _I64], _I64),
            "dsa_kpool_compress": ([_CFG, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P], _I),
            "dsa_kpool_compress_fp8": ([_CFG, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P], _I),
            "dsa_quantize_rows_fp8": ([_I64, _I, _P, _I, _P, _P, _P], _I),
            "dsa_k_norm": ([_I64, _I, _P, _P, _P, _F, _P], _I),
            "dsa_topk_to_mask": ([_I, _I, _I, _P, _P, _P], _I),
            "dsa_mla_masked_attn": ([_CFG, _I, _I, _I, _F, _P, _P, _P, _P, _I, _P, _I64, _P, _I,
                                     _I, _P, _P, _P], _I),
            "dsa_indexer_store": ([_I, _I, _I, _P, _P, _P, _P, _P, _P, _P], _I),
            "dsa_write_geom": ([_I, _P, _P, _P, _P], _I),
            "dsa_pool_append": ([_CFG, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P], _I),
            "dsa_compact_pools": ([_I, _I, _P, _P, _P, _P], _I),
            "dsa_index_scores": ([_CFG, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P, _I, _P, _P, _P,
                                  _P, _P, _P], _I),
            "dsa_compact_index_scores": ([_CFG, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P, _I, _P,
                                          _P, _P, _P, _P], _I),
            "dsa_topk_workspace": ([_CFG, _I, _I], _SZ),
            "dsa_topk_pools_workspace": ([_CFG, _I, _I], _SZ),
            "dsa_topk_pools": ([_CFG, _I, _I, _P, _P, _P, _P, _SZ, _P], _I),
            "dsa_expand_selection": ([_CFG, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P], _I),
            "dsa_topk_expand": ([_CFG, _I, _I, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _SZ,
                                 _P], _I),
            "dsa_sparse_mla_decode_workspace": ([_CFG, _I, _I], _SZ),
            "dsa_sparse_mla_decode": ([_CFG, _I, _I, _I, _F, _P, _P, _P, _P, _I, _P, _I64, _I,
                                       _P, _I, _I, _P, _P, _P, _SZ, _P], _I),
            "dsa_sparse_mla_decode_noalloc": ([_CFG, _I, _I, _I, _F, _P, _P, _P, _P, _I, _P,
                                               _I64, _I, _P, _I, _I, _P, _P, _P], _I),
            "dsa_stream_read": ([_P, _SZ, _P, _P], _I),
            "dsa_empty_launch": ([_I, _P], _I),
            "dsa_mfma_rate": ([_I, _I, _I, _P, _P], _I),
            "dsa_absorb_q": ([_CFG, _P, _SZ, _P, _SZ, _I, _I, _P, _SZ], _I),
            "dsa_absorb_o": ([_CFG, _P, _SZ, _P, _SZ, _I, _I, _P, _SZ], _I),
            "dsa_f32_to_bf16_rne": ([_P, _P, _SZ], None),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def last_error() -> str:
    return lib().dsa_last_error().decode()


def version() -> str:
    return lib().dsa_version().decode()


def _check(rc: int):
    if rc != 0:
        raise DsaError(rc, last_error())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name, dtypes, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must live on the GPU")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    return t


_FP8 = (torch.uint8, torch.float8_e4m3fn)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype in _FP8:
        return DSA_FP8_E4M3
    raise TypeError(f"unsupported data dtype {t.dtype}")


# ------------------------------------------------------------------ geometry

def config_validate(cfg: Config) -> int:
    return int(lib().dsa_config_validate(ctypes.byref(cfg)))


def select_k(cfg: Config, n_pools: int) -> int:
    v = int(lib().dsa_select_k(ctypes.byref(cfg), n_pools))
    _check(min(v, 0))
    return v


def out_width(cfg: Config) -> int:
    v = int(lib().dsa_out_width(ctypes.byref(cfg)))
    _check(min(v, 0))
    return v


def num_pools(S: int, first_key: int, kpool: int) -> int:
    v = int(lib().dsa_num_pools(S, first_key, kpool))
    _check(min(v, 0))
    return v


# ------------------------------------------------------------------ the six steps

def kpool_compress(cfg: Config, k, gate, ape, valid, first_key: int = 0, pool_keys=None,
                   pool_valid=None):
    """k, gate [B,S,D] bf16; ape [KP,D] f32; valid [B,S] u8 -> (pool_keys [B,P,D] bf16,
    pool_valid [B,P] u8)."""
    _dev(k, "k", (torch.bfloat16,))
    B, S, D = k.shape
    KP = cfg.index_kpool
    _dev(gate, "gate", (torch.bfloat16,), (B, S, D))
    _dev(ape, "ape", (torch.float32,), (KP, D))
    _dev(valid, "valid", (torch.uint8,), (B, S))
    if D != cfg.index_head_dim:
        raise ValueError("key width differs from index_head_dim")
    P = num_pools(S, first_key, KP)
    if pool_keys is None:
        pool_keys = torch.empty((B, P, D), dtype=torch.bfloat16, device=k.device)
    if pool_valid is None:
        pool_valid = torch.empty((B, P), dtype=torch.uint8, device=k.device)
    _dev(pool_keys, "pool_keys", (torch.bfloat16,), (B, P, D))
    _dev(pool_valid, "pool_valid", (torch.uint8,), (B, P))
    _check(lib().dsa_kpool_compress(ctypes.byref(cfg), B, S, first_key, _ptr(k), _ptr(gate),
                                    _ptr(ape), _ptr(valid), _ptr(pool_keys), _ptr(pool_valid),
                                    _stream(k)))
    return pool_keys, pool_valid


def kpool_compress_fp8(cfg: Config, k, gate, ape, valid, first_key: int = 0, pool_keys=None,
                       pool_key_scales=None, pool_valid=None):
    """kpool_compress with fp8 pooled keys: -> (pool_keys [B,P,D] uint8 e4m3 codes,
    pool_key_scales [B,P] f32, pool_valid [B,P] u8)."""
    _dev(k, "k", (torch.bfloat16,))
    B, S, D = k.shape
    KP = cfg.index_kpool
    _dev(gate, "gate", (torch.bfloat16,), (B, S, D))
    _dev(ape, "ape", (torch.float32,), (KP, D))
    _dev(valid, "valid", (torch.uint8,), (B, S))
    if D != cfg.index_head_dim:
        raise ValueError("key width differs from index_head_dim")
    P = num_pools(S, first_key, KP)
    if pool_keys is None:
        pool_keys = torch.empty((B, P, D), dtype=torch.uint8, device=k.device)
    if pool_key_scales is None:
        pool_key_scales = torch.empty((B, P), dtype=torch.float32, device=k.device)
    if pool_valid is None:
        pool_valid = torch.empty((B, P), dtype=torch.uint8, device=k.device)
    _dev(pool_keys, "pool_keys", _FP8, (B, P, D))
    _dev(pool_key_scales, "pool_key_scales", (torch.float32,), (B, P))
    _dev(pool_valid, "pool_valid", (torch.uint8,), (B, P))
    _check(lib().dsa_kpool_compress_fp8(ctypes.byref(cfg), B, S, first_key, _ptr(k), _ptr(gate),
                                        _ptr(ape), _ptr(valid), _ptr(pool_keys),
                                        _ptr(pool_key_scales), _ptr(pool_valid), _stream(k)))
    return pool_keys, pool_key_scales, pool_valid


def quantize_rows_fp8(src, codes=None, scales=None):
    """src [..., n] bf16 or f32 -> (codes uint8 [..., n] e4m3, scales f32 [...]), per row
    scale amax/448."""
    _dev(src, "src", (torch.bfloat16, torch.float32))
    n = src.shape[-1]
    rows = src.numel() // n if n else 0
    if codes is None:
        codes = torch.empty(src.shape, dtype=torch.uint8, device=src.device)
    if scales is None:
        scales = torch.empty(src.shape[:-1], dtype=torch.float32, device=src.device)
    _dev(codes, "codes", _FP8, tuple(src.shape))
    _dev(scales, "scales", (torch.float32,), tuple(src.shape[:-1]))
    code = DSA_F32 if src.dtype == torch.float32 else DSA_BF16
    _check(lib().dsa_quantize_rows_fp8(rows, n, _ptr(src), code, _ptr(codes), _ptr(scales),
                                       _stream(src)))
    return codes, scales


def k_norm(x, weight, bias, eps: float = 1e-5):
    """indexer.k_norm, a LayerNorm with a bias, in place on x [..., D] bf16; returns x."""
    _dev(x, "x", (torch.bfloat16,))
    D = x.shape[-1]
    _dev(weight, "weight", (torch.bfloat16,), (D,))
    _dev(bias, "bias", (torch.bfloat16,), (D,))
    rows = x.numel() // D if D else 0
    _check(lib().dsa_k_norm(rows, D, _ptr(x), _ptr(weight), _ptr(bias), float(eps), _stream(x)))
    return x


def indexer_store(pos, k_row, gate_row, k_cache, gate_cache, valid):
    """Staged rows k_row/gate_row [B,D] bf16 to position pos[b] of k_cache/gate_cache
    [B,S,D], marking valid [B,S]; all in place."""
    _dev(k_cache, "k_cache", (torch.bfloat16,))
    B, S, D = k_cache.shape
    _dev(gate_cache, "gate_cache", (torch.bfloat16,), (B, S, D))
    _dev(valid, "valid", (torch.uint8,), (B, S))
    _dev(pos, "pos", (torch.int32,), (B,))
    _dev(k_row, "k_row", (torch.bfloat16,), (B, D))
    _dev(gate_row, "gate_row", (torch.bfloat16,), (B, D))
    _check(lib().dsa_indexer_store(B, S, D, _ptr(pos), _ptr(k_row), _ptr(gate_row), _ptr(k_cache),
                                   _ptr(gate_cache), _ptr(valid), _stream(k_cache)))


def write_geom(seq_len, row_seq=None, row_pos=None):
    """Decode geometry from the live lengths: (row_seq [B], row_pos [B]) int32."""
    _dev(seq_len, "seq_len", (torch.int32,))
    B = seq_len.shape[0]
    if row_seq is None:
        row_seq = torch.empty((B,), dtype=torch.int32, device=seq_len.device)
    if row_pos is None:
        row_pos = torch.empty((B,), dtype=torch.int32, device=seq_len.device)
    _dev(row_seq, "row_seq", (torch.int32,), (B,))
    _dev(row_pos, "row_pos", (torch.int32,), (B,))
    _check(lib().dsa_write_geom(B, _ptr(seq_len), _ptr(row_seq), _ptr(row_pos), _stream(seq_len)))
    return row_seq, row_pos


def pool_append(cfg: Config, pos, k, gate, ape, valid, pool_keys, pool_valid, ids, n_valid, *,
                first_key: int, pool_key_scales=None):
    """The pool each sequence's new token (pos [B]) completes: key (bf16, or fp8 codes with
    pool_key_scales) and validity as kpool_compress computes them, and, when valid, its id
    appended to ids/n_valid. Everything is updated in place."""
    _dev(k, "k", (torch.bfloat16,))
    B, S, D = k.shape
    KP = cfg.index_kpool
    _dev(gate, "gate", (torch.bfloat16,), (B, S, D))
    _dev(ape, "ape", (torch.float32,), (KP, D))
    _dev(valid, "valid", (torch.uint8,), (B, S))
    _dev(pos, "pos", (torch.int32,), (B,))
    P = num_pools(S, first_key, KP)
    if pool_key_scales is None:
        _dev(pool_keys, "pool_keys", (torch.bfloat16,), (B, P, D))
    else:
        _dev(pool_keys, "pool_keys", _FP8, (B, P, D))
        _dev(pool_key_scales, "pool_key_scales", (torch.float32,), (B, P))
    _dev(pool_valid, "pool_valid", (torch.uint8,), (B, P))
    _dev(ids, "ids", (torch.int32,), (B, P))
    _dev(n_valid, "n_valid", (torch.int32,), (B,))
    _check(lib().dsa_pool_append(ctypes.byref(cfg), B, S, first_key, _ptr(pos), _ptr(k),
                                 _ptr(gate), _ptr(ape), _ptr(valid), _ptr(pool_keys),
                                 _ptr(pool_key_scales), _ptr(pool_valid), _ptr(ids),
                                 _ptr(n_valid), _stream(k)))


def compact_pools(pool_valid, ids=None, n_valid=None):
    """pool_valid [B,P] u8 -> (ids [B,P] i32, n_valid [B] i32)."""
    _dev(pool_valid, "pool_valid", (torch.uint8,))
    B, P = pool_valid.shape
    if ids is None:
        ids = torch.empty((B, P), dtype=torch.int32, device=pool_valid.device)
    if n_valid is None:
        n_valid = torch.empty((B,), dtype=torch.int32, device=pool_valid.device)
    _dev(ids, "ids", (torch.int32,), (B, P))
    _dev(n_valid, "n_valid", (torch.int32,), (B,))
    _check(lib().dsa_compact_pools(B, P, _ptr(pool_valid), _ptr(ids), _ptr(n_valid),
                                   _stream(pool_valid)))
    return ids, n_valid


def index_scores(cfg: Config, q, w, row_seq, row_pos, keys, ids, n_valid, *, first_key: int,
                 scale: float, key_scales=None, scores=None, cand=None):
    """q [Q,Hi,D] bf16; w [Q,Hi] f32; keys [B,P,D] bf16 or fp8 (+ key_scales [B,P] f32)
    -> (scores [Q,P] f32, cand [Q,P] u8)."""
    _dev(q, "q", (torch.bfloat16,))
    Q, Hi, D = q.shape
    _dev(w, "w", (torch.float32,), (Q, Hi))
    _dev(row_seq, "row_seq", (torch.int32,), (Q,))
    _dev(row_pos, "row_pos", (torch.int32,), (Q,))
    _dev(keys, "keys", (torch.bfloat16,) + _FP8)
    B, P, Dk = keys.shape
    if Dk != D or D != cfg.index_head_dim or Hi != cfg.index_heads:
        raise ValueError("q / keys shapes differ from the config's indexer geometry")
    code = _dtype_code(keys)
    if code == DSA_FP8_E4M3:
        _dev(key_scales, "key_scales", (torch.float32,), (B, P))
    _dev(ids, "ids", (torch.int32,), (B, P))
    _dev(n_valid, "n_valid", (torch.int32,), (B,))
    if scores is None:
        scores = torch.empty((Q, P), dtype=torch.float32, device=q.device)
    if cand is None:
        cand = torch.empty((Q, P), dtype=torch.uint8, device=q.device)
    _dev(scores, "scores", (torch.float32,), (Q, P))
    _dev(cand, "cand", (torch.uint8,), (Q, P))
    _check(lib().dsa_index_scores(ctypes.byref(cfg), Q, B, P, first_key, float(scale), _ptr(q),
                                  _ptr(w), _ptr(row_seq), _ptr(row_pos), _ptr(keys), code,
                                  _ptr(key_scales) if code == DSA_FP8_E4M3 else None, _ptr(ids),
                                  _ptr(n_valid), _ptr(scores), _ptr(cand), _stream(q)))
    return scores, cand


def compact_index_scores(cfg: Config, q, w, row_seq, row_pos, keys, pool_valid, *,
                         first_key: int, scale: float, key_scales=None, scores=None, cand=None):
    """compact_pools + index_scores in one launch: q [Q,Hi,D] bf16; w [Q,Hi] f32; keys
    [B,P,D] bf16 or fp8 (+ key_scales [B,P] f32); pool_valid [B,P] u8
    -> (scores [Q,P] f32, cand [Q,P] u8), equal to index_scores on compact_pools' list."""
    _dev(q, "q", (torch.bfloat16,))
    Q, Hi, D = q.shape
    _dev(w, "w", (torch.float32,), (Q, Hi))
    _dev(row_seq, "row_seq", (torch.int32,), (Q,))
    _dev(row_pos, "row_pos", (torch.int32,), (Q,))
    _dev(keys, "keys", (torch.bfloat16,) + _FP8)
    B, P, Dk = keys.shape
    if Dk != D or D != cfg.index_head_dim or Hi != cfg.index_heads:
        raise ValueError("q / keys shapes differ from the config's indexer geometry")
    code = _dtype_code(keys)
    if code == DSA_FP8_E4M3:
        _dev(key_scales, "key_scales", (torch.float32,), (B, P))
    _dev(pool_valid, "pool_valid", (torch.uint8,), (B, P))
    if scores is None:
        scores = torch.empty((Q, P), dtype=torch.float32, device=q.device)
    if cand is None:
        cand = torch.empty((Q, P), dtype=torch.uint8, device=q.device)
    _dev(scores, "scores", (torch.float32,), (Q, P))
    _dev(cand, "cand", (torch.uint8,), (Q, P))
    _check(lib().dsa_compact_index_scores(ctypes.byref(cfg), Q, B, P, first_key, float(scale),
                                          _ptr(q), _ptr(w), _ptr(row_seq), _ptr(row_pos),
                                          _ptr(keys), code,
                                          _ptr(key_scales) if code == DSA_FP8_E4M3 else None,
                                          _ptr(pool_valid), _ptr(scores), _ptr(cand), _stream(q)))
    return scores, cand


def topk_workspace(cfg: Config, Q: int, P: int) -> int:
    """Bytes of the top-k workspace (0: one block a row, no workspace used)."""
    return int(lib().dsa_topk_workspace(ctypes.byref(cfg), Q, P))


def _topk_ws(cfg, Q, P, ws, device):
    """The caller's workspace, or a fresh one of the size the call can use (None if 0);
    ws=False asks for the one-block-a-row selection."""
    if ws is False:
        return None, 0
    if ws is None:
        need = topk_workspace(cfg, Q, P)
        ws = torch.empty((need,), dtype=torch.uint8, device=device) if need else None
    return ws, (0 if ws is None else ws.numel() * ws.element_size())


def topk_pools(cfg: Config, scores, cand, sel=None, ws=None):
    """scores [Q,P] f32, cand [Q,P] u8 -> sel [Q, select_k(P)] i32 (ascending, -1 padded)."""
    _dev(scores, "scores", (torch.float32,))
    Q, P = scores.shape
    _dev(cand, "cand", (torch.uint8,), (Q, P))
    kw = select_k(cfg, P)
    if sel is None:
        sel = torch.empty((Q, kw), dtype=torch.int32, device=scores.device)
    _dev(sel, "sel", (torch.int32,), (Q, kw))
    ws, ws_bytes = _topk_ws(cfg, Q, P, ws, scores.device)
    _check(lib().dsa_topk_pools(ctypes.byref(cfg), Q, P, _ptr(scores), _ptr(cand), _ptr(sel),
                                _ptr(ws), ws_bytes, _stream(scores)))
    return sel


def expand_selection(cfg: Config, sel, row_seq, row_pos, valid, *, S: int, first_key: int,
                     token_ids=None):
    """sel [Q,Kw] i32 -> token_ids [Q, out_width] i32. valid [B,S] u8 (read for the tail)."""
    _dev(sel, "sel", (torch.int32,))
    Q, kw = sel.shape
    _dev(row_seq, "row_seq", (torch.int32,), (Q,))
    _dev(row_pos, "row_pos", (torch.int32,), (Q,))
    _dev(valid, "valid", (torch.uint8,))
    B = valid.shape[0]
    if valid.shape[1] != S:
        raise ValueError("valid must be [B, S]")
    W = out_width(cfg)
    if token_ids is None:
        token_ids = torch.empty((Q, W), dtype=torch.int32, device=sel.device)
    _dev(token_ids, "token_ids", (torch.int32,), (Q, W))
    _check(lib().dsa_expand_selection(ctypes.byref(cfg), Q, kw, B, S, first_key, _ptr(sel),
                                      _ptr(row_seq), _ptr(row_pos), _ptr(valid), _ptr(token_ids),
                                      _stream(sel)))
    return token_ids


def topk_expand(cfg: Config, scores, cand, row_seq, row_pos, valid, *, S: int, first_key: int,
                sel=None, token_ids=None, ws=None):
    """Fused top-k and expansion: the same (sel, token_ids) as topk_pools then
    expand_selection. scores/cand [Q,P]; valid [B,S] u8 (read for the tail)."""
    _dev(scores, "scores", (torch.float32,))
    Q, P = scores.shape
    _dev(cand, "cand", (torch.uint8,), (Q, P))
    _dev(row_seq, "row_seq", (torch.int32,), (Q,))
    _dev(row_pos, "row_pos", (torch.int32,), (Q,))
    _dev(valid, "valid", (torch.uint8,))
    B = valid.shape[0]
    if valid.shape[1] != S:
        raise ValueError("valid must be [B, S]")
    kw = select_k(cfg, P)
    W = out_width(cfg)
    if sel is None:
        sel = torch.empty((Q, kw), dtype=torch.int32, device=scores.device)
    if token_ids is None:
        token_ids = torch.empty((Q, W), dtype=torch.int32, device=scores.device)
    _dev(sel, "sel", (torch.int32,), (Q, kw))
    _dev(token_ids, "token_ids", (torch.int32,), (Q, W))
    ws, ws_bytes = _topk_ws(cfg, Q, P, ws, scores.device)
    _check(lib().dsa_topk_expand(ctypes.byref(cfg), Q, P, _ptr(scores), _ptr(cand), B, S,
                                 first_key, _ptr(row_seq), _ptr(row_pos), _ptr(valid), _ptr(sel),
                                 _ptr(token_ids), _ptr(ws), ws_bytes, _stream(scores)))
    return sel, token_ids


def sparse_mla_workspace(cfg: Config, Q: int, W: int) -> int:
    return int(lib().dsa_sparse_mla_decode_workspace(ctypes.byref(cfg), Q, W))


def _mla_args(cfg: Config, q_abs, token_ids, row_seq, kv, B, kv_scales, block_table, out, lse):
    _dev(q_abs, "q_abs", (torch.bfloat16,))
    Q, H, C = q_abs.shape
    if H != cfg.heads or C != 512:
        raise ValueError("q_abs must be [Q, heads, 512]")
    _dev(token_ids, "token_ids", (torch.int32,))
    if token_ids.shape[0] != Q:
        raise ValueError("token_ids rows differ from q_abs rows")
    W = token_ids.shape[1]
    _dev(row_seq, "row_seq", (torch.int32,), (Q,))
    _dev(kv, "kv", (torch.bfloat16,) + _FP8)
    if kv.shape[-1] != 512:
        raise ValueError("kv rows must be 512 wide")
    rows = kv.numel() // 512
    code = _dtype_code(kv)
    if code == DSA_FP8_E4M3:
        _dev(kv_scales, "kv_scales", (torch.float32,))
        if kv_scales.numel() != rows:
            raise ValueError("kv_scales must hold one scale per latent row")
    max_blocks = 0
    if block_table is not None:
        _dev(block_table, "block_table", (torch.int32,))
        if block_table.shape[0] != B:
            raise ValueError("block_table must be [B, max_blocks]")
        max_blocks = block_table.shape[1]
    if out is None:
        out = torch.empty((Q, H, 512), dtype=torch.float32, device=q_abs.device)
    if lse is None:
        lse = torch.empty((Q, H), dtype=torch.float32, device=q_abs.device)
    _dev(out, "out", (torch.float32,), (Q, H, 512))
    _dev(lse, "lse", (torch.float32,), (Q, H))
    return Q, W, rows, code, max_blocks, out, lse


def sparse_mla_decode(cfg: Config, q_abs, token_ids, row_seq, kv, *, B: int, sm_scale: float,
                      S: int, kv_scales=None, block_table=None, block_size: int = 64,
                      out=None, lse=None, ws=None):
    """q_abs [Q,H,512] bf16; token_ids [Q,W] i32; kv [rows,512] bf16 or fp8 (+ kv_scales
    [rows] f32); contiguous rows b*S + t (S > 0 required), or paged through block_table
    [B, max_blocks] (S > 0 also bounds the token ids; 0 = no bound).
    Returns (out [Q,H,512] f32, lse [Q,H] f32)."""
    Q, W, rows, code, max_blocks, out, lse = _mla_args(cfg, q_abs, token_ids, row_seq, kv, B,
                                                       kv_scales, block_table, out, lse)
    need = sparse_mla_workspace(cfg, Q, W)
    if need and ws is None:
        ws = torch.empty((need,), dtype=torch.uint8, device=q_abs.device)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().dsa_sparse_mla_decode(ctypes.byref(cfg), Q, W, B, float(sm_scale), _ptr(q_abs),
                                       _ptr(token_ids), _ptr(row_seq), _ptr(kv), code,
                                       _ptr(kv_scales) if code == DSA_FP8_E4M3 else None, rows,
                                       S, _ptr(block_table), max_blocks, block_size, _ptr(out),
                                       _ptr(lse), _ptr(ws), ws_bytes, _stream(q_abs)))
    return out, lse


def sparse_mla_decode_noalloc(cfg: Config, q_abs, token_ids, row_seq, kv, *, B: int,
                              sm_scale: float, S: int, kv_scales=None, block_table=None,
                              block_size: int = 64, out=None, lse=None):
    """sparse_mla_decode with the split partials in the library's fixed device scratch: pass
    out and lse to allocate nothing at all. Refuses (DSA_ERR_WORKSPACE) a shape whose
    partials exceed the scratch."""
    Q, W, rows, code, max_blocks, out, lse = _mla_args(cfg, q_abs, token_ids, row_seq, kv, B,
                                                       kv_scales, block_table, out, lse)
    _check(lib().dsa_sparse_mla_decode_noalloc(
        ctypes.byref(cfg), Q, W, B, float(sm_scale), _ptr(q_abs), _ptr(token_ids), _ptr(row_seq),
        _ptr(kv), code, _ptr(kv_scales) if code == DSA_FP8_E4M3 else None, rows, S,
        _ptr(block_table), max_blocks, block_size, _ptr(out), _ptr(lse), _stream(q_abs)))
    return out, lse


def topk_to_mask(token_ids, S: int, mask=None):
    """[Q, W] token ids -> [Q, S] u8 mask of the tokens present."""
    _dev(token_ids, "token_ids", (torch.int32,))
    Q, W = token_ids.shape
    if mask is None:
        mask = torch.empty((Q, S), dtype=torch.uint8, device=token_ids.device)
    _dev(mask, "mask", (torch.uint8,), (Q, S))
    _check(lib().dsa_topk_to_mask(Q, W, S, _ptr(token_ids), _ptr(mask), _stream(token_ids)))
    return mask


def mla_masked_attn(cfg: Config, q_abs, mask, row_seq, kv, *, B: int, sm_scale: float,
                    kv_scales=None, block_table=None, block_size: int = 64, out=None, lse=None):
    """Dense attention over every masked token (the cross-check of sparse_mla_decode): q_abs
    [Q,H,512] bf16; mask [Q,S] u8; kv as sparse_mla_decode with S = mask width."""
    _dev(q_abs, "q_abs", (torch.bfloat16,))
    Q, H, C = q_abs.shape
    if H != cfg.heads or C != 512:
        raise ValueError("q_abs must be [Q, heads, 512]")
    _dev(mask, "mask", (torch.uint8,))
    S = mask.shape[1]
    _dev(row_seq, "row_seq", (torch.int32,), (Q,))
    _dev(kv, "kv", (torch.bfloat16,) + _FP8)
    rows = kv.numel() // 512
    code = _dtype_code(kv)
    if code == DSA_FP8_E4M3:
        _dev(kv_scales, "kv_scales", (torch.float32,))
    max_blocks = 0
    if block_table is not None:
        _dev(block_table, "block_table", (torch.int32,))
        max_blocks = block_table.shape[1]
    if out is None:
        out = torch.empty((Q, H, 512), dtype=torch.float32, device=q_abs.device)
    if lse is None:
        lse = torch.empty((Q, H), dtype=torch.float32, device=q_abs.device)
    _check(lib().dsa_mla_masked_attn(ctypes.byref(cfg), Q, S, B, float(sm_scale), _ptr(q_abs),
                                     _ptr(mask), _ptr(row_seq), _ptr(kv), code,
                                     _ptr(kv_scales) if code == DSA_FP8_E4M3 else None, rows,
                                     _ptr(block_table), max_blocks, block_size, _ptr(out),
                                     _ptr(lse), _stream(q_abs)))
    return out, lse


# ------------------------------------------------------------------ host weight prep

def _host_f32(a, name):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def absorb_q(cfg: Config, q_b, kv_b, *, full_heads: int, threads: int = 0) -> np.ndarray:
    """Host f32 (numpy) -> q_absorb [full_heads*kv_lora_rank, q_lora_rank]."""
    q_b, pq = _host_f32(q_b, "q_b")
    kv_b, pk = _host_f32(kv_b, "kv_b")
    n = full_heads * cfg.kv_lora_rank * cfg.q_lora_rank
    out = np.zeros(max(n, 1), np.float32)
    _check(lib().dsa_absorb_q(ctypes.byref(cfg), pq, q_b.size, pk, kv_b.size, full_heads, threads,
                              out.ctypes.data_as(ctypes.c_void_p), n))
    return out[:n].reshape(full_heads * cfg.kv_lora_rank, cfg.q_lora_rank)


def absorb_o(cfg: Config, o_local, kv_b_local, *, local_heads: int, threads: int = 0) -> np.ndarray:
    """Host f32 (numpy) -> o_absorb [hidden, local_heads*kv_lora_rank]."""
    o_local, po = _host_f32(o_local, "o_local")
    kv_b_local, pk = _host_f32(kv_b_local, "kv_b_local")
    n = cfg.hidden * local_heads * cfg.kv_lora_rank
    out = np.zeros(max(n, 1), np.float32)
    _check(lib().dsa_absorb_o(ctypes.byref(cfg), po, o_local.size, pk, kv_b_local.size,
                              local_heads, threads, out.ctypes.data_as(ctypes.c_void_p), n))
    return out[:n].reshape(cfg.hidden, local_heads * cfg.kv_lora_rank)


def f32_to_bf16_rne(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros(x.shape, np.uint16)
    lib().dsa_f32_to_bf16_rne(x.ctypes.data_as(ctypes.c_void_p),
                              out.ctypes.data_as(ctypes.c_void_p), x.size)
    return out


def stream_read(buf, sink=None):
    """Measurement only: read every byte of the device tensor buf once (16-byte aligned, a
    multiple of 16 bytes); the XOR of its 32-bit words is folded into sink (uint32 [1])."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.zeros((1,), dtype=torch.int32, device=buf.device)
    _check(lib().dsa_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(buf)))
    return sink


def empty_launch(blocks: int = 1, stream=None):
    """Measurement only: one launch of a kernel that does nothing (blocks of 64 threads)."""
    st = stream if stream is not None else torch.cuda.current_stream()
    _check(lib().dsa_empty_launch(int(blocks), ctypes.c_void_p(st.cuda_stream)))


# Floating-point operations of one MFMA of each dsa_mfma_rate shape (2*M*N*K).
MFMA_RATE_SHAPES = {0: ("v_mfma_f32_32x32x16_bf16", 2 * 32 * 32 * 16),
                    1: ("v_mfma_f32_16x16x32_bf16", 2 * 16 * 16 * 32),
                    2: ("v_mfma_scale_f32_16x16x128_f8f6f4 (e4m3)", 2 * 16 * 16 * 128)}


def mfma_rate(kind: int, blocks: int, iters: int, out):
    """Measurement only: blocks x 4 waves x iters rounds of 4 independent MFMAs of one shape
    (MFMA_RATE_SHAPES); out: [blocks * 256] f32 on the device. Returns the flop count."""
    _dev(out, "out", (torch.float32,), (blocks * 256,))
    _check(lib().dsa_mfma_rate(int(kind), int(blocks), int(iters), _ptr(out), _stream(out)))
    return blocks * 4 * iters * 4 * MFMA_RATE_SHAPES[kind][1]

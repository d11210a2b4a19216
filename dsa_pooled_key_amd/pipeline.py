"""The decode step as one object: device buffers plus the launch sequence.

``DecodeStep`` owns the intermediate and output buffers of one batch and issues
compact_pools -> index_scores -> topk_pools -> expand_selection -> sparse_mla_decode on the
current stream through the C ABI (fused: compact_index_scores -> topk_expand ->
sparse_mla_decode, three launches of the same steps). It allocates only in its constructor, so ``run()`` can be
recorded into a HIP graph (``torch.cuda.CUDAGraph``) and replayed.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import binding as dsa
from .synth import DecodeInputs, Workload


def config_for(wl: Workload) -> dsa.Config:
    return dsa.Config.make(index_heads=wl.index_heads, index_head_dim=wl.index_dim,
                           index_kpool=wl.kpool, index_topk=wl.topk, heads=wl.heads,
                           always_select_tail=wl.tail)


def _bf16(a, dev):
    return torch.from_numpy(a.view("int16")).to(dev).view(torch.bfloat16)


def _t(a, dev):
    return None if a is None else torch.from_numpy(a).to(dev)


@dataclasses.dataclass
class DeviceDecodeInputs:
    """DecodeInputs copied to the GPU (bf16 as torch.bfloat16, fp8 as uint8 codes)."""
    pool_valid: torch.Tensor
    valid: torch.Tensor
    keys: torch.Tensor
    key_scales: Optional[torch.Tensor]
    q: torch.Tensor
    w: torch.Tensor
    row_seq: torch.Tensor
    row_pos: torch.Tensor
    q_abs: torch.Tensor
    kv: torch.Tensor
    kv_scales: Optional[torch.Tensor]
    block_table: Optional[torch.Tensor]

    @staticmethod
    def upload(di: DecodeInputs, dev="cuda") -> "DeviceDecodeInputs":
        keys = _t(di.keys, dev) if di.wl.key_fp8 else _bf16(di.keys, dev)
        kv = _t(di.kv, dev) if di.wl.kv_fp8 else _bf16(di.kv, dev)
        return DeviceDecodeInputs(
            pool_valid=_t(di.pool_valid, dev), valid=_t(di.valid, dev), keys=keys,
            key_scales=_t(di.key_scales, dev), q=_bf16(di.q, dev), w=_t(di.w, dev),
            row_seq=_t(di.row_seq, dev), row_pos=_t(di.row_pos, dev), q_abs=_bf16(di.q_abs, dev),
            kv=kv, kv_scales=_t(di.kv_scales, dev), block_table=_t(di.block_table, dev))


class DecodeStep:
    """One decode (or prefill-chunk) pass of the selection chain and the sparse MLA."""

    def __init__(self, wl: Workload, x: DeviceDecodeInputs, scale: float, sm_scale: float,
                 fused: bool = True):
        """fused: compaction and scoring in one launch (dsa_compact_index_scores) and top-k
        with token-id expansion in one launch (dsa_topk_expand); otherwise the five entry
        points in sequence. Both give the same scores, cand, sel and token_ids."""
        self.wl, self.x, self.scale, self.sm_scale = wl, x, scale, sm_scale
        self.fused = fused
        self.cfg = config_for(wl)
        dev = x.q.device
        B, P, Q = wl.B, wl.pools, wl.Q
        self.kw = dsa.select_k(self.cfg, P)
        self.width = dsa.out_width(self.cfg)
        self.ids = torch.empty((B, P), dtype=torch.int32, device=dev)
        self.n_valid = torch.empty((B,), dtype=torch.int32, device=dev)
        self.scores = torch.empty((Q, P), dtype=torch.float32, device=dev)
        self.cand = torch.empty((Q, P), dtype=torch.uint8, device=dev)
        self.sel = torch.empty((Q, self.kw), dtype=torch.int32, device=dev)
        self.token_ids = torch.empty((Q, self.width), dtype=torch.int32, device=dev)
        self.out = torch.empty((Q, wl.heads, 512), dtype=torch.float32, device=dev)
        self.lse = torch.empty((Q, wl.heads), dtype=torch.float32, device=dev)
        tk = dsa.topk_workspace(self.cfg, Q, P)
        self.topk_ws = torch.empty((tk,), dtype=torch.uint8, device=dev) if tk else None
        need = dsa.sparse_mla_workspace(self.cfg, Q, self.width)
        self.ws = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)

    def select(self):
        self.score()
        self.topk()

    def score(self):
        x, wl = self.x, self.wl
        if self.fused:
            dsa.compact_index_scores(self.cfg, x.q, x.w, x.row_seq, x.row_pos, x.keys,
                                     x.pool_valid, first_key=wl.first_key, scale=self.scale,
                                     key_scales=x.key_scales, scores=self.scores, cand=self.cand)
        else:
            dsa.compact_pools(x.pool_valid, self.ids, self.n_valid)
            dsa.index_scores(self.cfg, x.q, x.w, x.row_seq, x.row_pos, x.keys, self.ids,
                             self.n_valid, first_key=wl.first_key, scale=self.scale,
                             key_scales=x.key_scales, scores=self.scores, cand=self.cand)

    def topk(self):
        x, wl = self.x, self.wl
        if self.fused:
            dsa.topk_expand(self.cfg, self.scores, self.cand, x.row_seq, x.row_pos, x.valid,
                            S=wl.S, first_key=wl.first_key, sel=self.sel, token_ids=self.token_ids,
                            ws=self.topk_ws if self.topk_ws is not None else False)
        else:
            dsa.topk_pools(self.cfg, self.scores, self.cand, self.sel,
                           ws=self.topk_ws if self.topk_ws is not None else False)
            dsa.expand_selection(self.cfg, self.sel, x.row_seq, x.row_pos, x.valid, S=wl.S,
                                 first_key=wl.first_key, token_ids=self.token_ids)

    def attend(self):
        x, wl = self.x, self.wl
        dsa.sparse_mla_decode(self.cfg, x.q_abs, self.token_ids, x.row_seq, x.kv, B=wl.B,
                              sm_scale=self.sm_scale, S=wl.S, kv_scales=x.kv_scales,
                              block_table=x.block_table, out=self.out, lse=self.lse, ws=self.ws)

    def run(self):
        self.select()
        self.attend()

"""dsa_sparse_mla_decode_noalloc, the sparse MLA entry point for callers that cannot allocate:
its split partials live in the library's fixed device scratch. Calls in a row on one GPU, each
smaller than the one before (so stale partials of a larger call sit in the scratch), give
outputs bit-identical to dsa_sparse_mla_decode with its own workspace, and within the parity
rules of the oracle; a shape whose partials exceed the scratch is refused before anything
runs, leaving the outputs untouched."""
import numpy as np
import pytest
import torch

import oracle
from dsa_pooled_key_amd import binding as dsa
from dsa_pooled_key_amd import synth
from dsa_pooled_key_amd.pipeline import DeviceDecodeInputs, config_for
from tests import checks

pytestmark = pytest.mark.gpu

SCRATCH = 16 << 20


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _one_call(name):
    di = synth.make_decode_inputs(name)
    wl = di.wl
    x = DeviceDecodeInputs.upload(di)
    cfg = config_for(wl)
    tok = synth.draw_token_ids(di)
    need = dsa.sparse_mla_workspace(cfg, wl.Q, tok.shape[1])
    assert 0 < need <= SCRATCH, (name, need)
    kw = dict(B=wl.B, sm_scale=di.sm_scale, S=wl.S, kv_scales=x.kv_scales,
              block_table=x.block_table)
    out = torch.full((wl.Q, wl.heads, 512), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((wl.Q, wl.heads), 7.0, dtype=torch.float32, device="cuda")
    print(f"[noalloc] {name}: Q={wl.Q} W={tok.shape[1]} partials {need} B", flush=True)
    dsa.sparse_mla_decode_noalloc(cfg, x.q_abs, _dev(tok), x.row_seq, x.kv, out=out, lse=lse, **kw)
    ro_ws, rl_ws = dsa.sparse_mla_decode(cfg, x.q_abs, _dev(tok), x.row_seq, x.kv, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, ro_ws) and torch.equal(lse, rl_ws)
    rows = np.unique(np.r_[0, wl.Q // 2, wl.Q - 1])
    ro, rl = oracle.sparse_mla(di.q_abs[rows], tok[rows], di.row_seq[rows], di.kv,
                               sm_scale=di.sm_scale, S=wl.S, kv_scales=di.kv_scales,
                               block_table=di.block_table)
    checks.check_mla(out.cpu().numpy()[rows], lse.cpu().numpy()[rows], ro, rl, wl.kv_fp8)
    return need


def test_noalloc_calls_in_a_row_equal_the_workspace_entry_point():
    sizes = [_one_call(n) for n in ("fp8_mixed_b32", "decode_b8_32k", "ragged_fp8")]
    assert sizes[0] > sizes[1] > sizes[2]


def test_noalloc_refuses_partials_beyond_the_scratch():
    S, W, H, Q = 40000, 32768, 32, 64
    cfg = dsa.Config.make(index_heads=32, index_head_dim=128, index_kpool=4, index_topk=W,
                          heads=H)
    assert dsa.sparse_mla_workspace(cfg, Q, W) > SCRATCH
    kv = torch.zeros((S, 512), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((Q, H, 512), dtype=torch.bfloat16, device="cuda")
    tok = torch.zeros((Q, W), dtype=torch.int32, device="cuda")
    rs = torch.zeros((Q,), dtype=torch.int32, device="cuda")
    out = torch.full((Q, H, 512), 3.0, dtype=torch.float32, device="cuda")
    lse = torch.full((Q, H), 3.0, dtype=torch.float32, device="cuda")
    with pytest.raises(dsa.DsaError) as e:
        dsa.sparse_mla_decode_noalloc(cfg, q, tok, rs, kv, B=1, sm_scale=0.0625, S=S, out=out,
                                      lse=lse)
    assert e.value.code == -12 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0) and torch.all(lse == 3.0)

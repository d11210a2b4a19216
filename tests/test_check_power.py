"""The parity rules of tests/checks.py can fail: on the CPU, with the oracle's own outputs
deliberately damaged, each rule rejects a plausible mistake of the GPU path and accepts the
rounding the GPU path legitimately adds.

* sparse MLA over 4,096 fp8 latent rows (the graded decode's selection width) split in 16
  parts of 256 like the GPU's plan: an output scaled by 0.9 and an output with one split's
  tokens dropped both fail; the element-wise rule alone would have accepted them. Outputs
  rounded the way the GPU rounds (bf16 P operand, bf16 split partials) pass.
* index scores: one head dropped, two heads' weights swapped, a 0.3% scale error all fail; the
  same scores computed in f32 in another summation order pass.
* selections: a pool swapped far from the cutoff fails; equal scores at the cutoff pass.
"""
import numpy as np
import pytest

import oracle
from dsa_pooled_key_amd import synth
from tests import checks

N_LAT, W, H, Q = 8192, 4096, 32, 2


def _bf(x):
    return synth.bf16_to_f32(synth.bf16_bits(np.asarray(x, np.float32))).astype(np.float64)


@pytest.fixture(scope="module", params=[0.5, synth.PEAKED_QABS_STD], ids=["uniform", "peaked"])
def mla_case(request):
    rng = np.random.default_rng(5)
    kv, sc = synth.e4m3_quantize_rows(rng.normal(0.0, 0.5, (N_LAT, 512)).astype(np.float32))
    q = synth.bf16_bits(rng.normal(0.0, request.param, (Q, H, 512)).astype(np.float32))
    tok = np.stack([np.sort(rng.choice(N_LAT, W, replace=False)) for _ in range(Q)]).astype(np.int32)
    rs = np.zeros(Q, np.int32)
    ro, rl = oracle.sparse_mla(q, tok, rs, kv, sm_scale=synth.SM_SCALE, S=N_LAT, kv_scales=sc)
    return kv, sc, q, tok, rs, ro, rl


def _gpu_like(kv, sc, q, tok):
    """The GPU plan's rounding, in numpy: splits of 256 slots, P = exp(l - m_split) in bf16,
    each split's unnormalised output in bf16, the merge in f32."""
    v_all = checks.e4m3_lut()[kv] * sc[:, None].astype(np.float64)
    qf = synth.bf16_to_f32(q).astype(np.float64)
    out = np.zeros((Q, H, 512))
    for r in range(Q):
        v = v_all[tok[r]]
        l = (qf[r] @ v.T) * synth.SM_SCALE
        m = l.max(1, keepdims=True)
        O = np.zeros((H, 512))
        L = np.zeros((H, 1))
        for s in range(0, W, 256):
            ls = l[:, s:s + 256]
            ms = ls.max(1, keepdims=True)
            p = _bf(np.exp(ls - ms))
            a = np.exp(ms - m)
            O += a * _bf(p @ v[s:s + 256])
            L += a * p.sum(1, keepdims=True)
        out[r] = O / L
    return out.astype(np.float32)


def test_mla_rule_accepts_the_gpu_plans_rounding(mla_case):
    kv, sc, q, tok, rs, ro, rl = mla_case
    rmax, rl2 = checks.check_mla(_gpu_like(kv, sc, q, tok), rl, ro, rl, fp8=True)
    assert rmax < 5e-3 and rl2 < 5e-3


def test_mla_rule_rejects_a_scaled_output(mla_case):
    kv, sc, q, tok, rs, ro, rl = mla_case
    bad = (0.9 * ro).astype(np.float32)
    with pytest.raises(AssertionError):
        checks.check_mla(bad, rl, ro, rl, fp8=True)
    rmax, rl2 = checks.mla_errors(bad, ro, rl)
    assert rmax.min() > 0.09 and rl2.min() > 0.09
    if np.abs(ro).max() < 0.1:        # nearly uniform softmax: the element-wise rule passes it
        assert (np.abs(bad - ro) - (5e-2 + 1e-2 * np.abs(ro))).max() <= 0


@pytest.mark.parametrize("split", [0, 7, 15])
def test_mla_rule_rejects_a_dropped_split(mla_case, split):
    kv, sc, q, tok, rs, ro, rl = mla_case
    t2 = tok.copy()
    t2[:, split * 256:(split + 1) * 256] = -1
    bo, bl = oracle.sparse_mla(q, t2, rs, kv, sm_scale=synth.SM_SCALE, S=N_LAT, kv_scales=sc)
    with pytest.raises(AssertionError):
        checks.check_mla(bo.astype(np.float32), rl, ro, rl, fp8=True)
    # even with a matching lse, the per-head output rule flags most heads (a peaked head whose
    # weight sits outside the dropped split may barely move)
    rmax, rl2 = checks.mla_errors(bo, ro, rl)
    assert (np.maximum(rmax, rl2) > 1e-2).mean() > 0.75 and rmax.max() > 5e-2
    with pytest.raises(AssertionError):
        checks.check_mla(bo.astype(np.float32), bl, ro, bl, fp8=True)


def test_mla_rule_zero_rows():
    ro = np.zeros((1, 2, 512))
    rl = np.full((1, 2), -np.inf)
    checks.check_mla(np.zeros((1, 2, 512), np.float32), rl, ro, rl, fp8=False)
    bad = np.zeros((1, 2, 512), np.float32)
    bad[0, 1, 3] = 1e-3
    with pytest.raises(AssertionError):
        checks.check_mla(bad, rl, ro, rl, fp8=False)


# ---------------------------------------------------------------------- scores and selection

@pytest.fixture(scope="module", params=[False, True], ids=["bf16", "fp8"])
def score_case(request):
    fp8 = request.param
    rng = np.random.default_rng(9)
    B, P, Hi, D, R = 2, 3000, 32, 128, 3
    kf = synth.layer_norm_f32(rng.standard_normal((B, P, D)).astype(np.float32))
    if fp8:
        keys, ks = synth.e4m3_quantize_rows(kf)
    else:
        keys, ks = synth.bf16_bits(kf), None
    q = synth.bf16_bits(rng.standard_normal((R, Hi, D)).astype(np.float32))
    w = (rng.standard_normal((R, Hi)) * Hi ** -0.5).astype(np.float32)
    row_seq = np.array([0, 1, 1], np.int32)
    row_pos = np.array([P * 4 - 1, P * 4 - 1, 5000], np.int32)
    pv = (rng.random((B, P)) < 0.9).astype(np.uint8)
    ids, nv = oracle.compact_pools(pv)
    scale = float(np.float32(D ** -0.5))
    rs, rc = oracle.index_scores(q, w, row_seq, row_pos, keys, ids, nv, kpool=4, first_key=0,
                                 scale=scale, key_scales=ks)
    bound = checks.score_error_bound(q, w, row_seq, keys, ks, scale)
    return q, w, row_seq, keys, ks, scale, rs, rc, bound


def _f32_scores(q, w, row_seq, keys, ks, scale, rc, drop=None, swap=None):
    """The scores in binary32 in another order (BLAS dot products, heads summed last to
    first), optionally with one head dropped or two heads' weights swapped."""
    kv = checks.key_values(keys, ks).astype(np.float32)
    qf = synth.bf16_to_f32(q)
    out = np.full(rc.shape, -np.inf, np.float32)
    for r in range(q.shape[0]):
        wr = w[r].copy()
        if swap is not None:
            wr[list(swap)] = wr[list(swap[::-1])]
        x = np.maximum((qf[r] @ kv[row_seq[r]].T) * np.float32(scale), np.float32(0))   # [Hi,P]
        acc = np.zeros(x.shape[1], np.float32)
        for h in range(x.shape[0] - 1, -1, -1):
            if h != drop:
                acc = acc + wr[h] * x[h]
        out[r] = np.where(rc[r] == 1, acc, -np.inf)
    return out


def test_score_rule_accepts_another_f32_order(score_case):
    q, w, row_seq, keys, ks, scale, rs, rc, bound = score_case
    checks.check_scores(_f32_scores(q, w, row_seq, keys, ks, scale, rc), rs, rc, bound)


@pytest.mark.parametrize("damage", ["drop", "swap", "scale"])
def test_score_rule_rejects_damage(score_case, damage):
    q, w, row_seq, keys, ks, scale, rs, rc, bound = score_case
    if damage == "drop":
        bad = _f32_scores(q, w, row_seq, keys, ks, scale, rc, drop=17)
    elif damage == "swap":
        bad = _f32_scores(q, w, row_seq, keys, ks, scale, rc, swap=(3, 4))
    else:
        bad = _f32_scores(q, w, row_seq, keys, ks, scale, rc) * np.float32(1.003)
    with pytest.raises(AssertionError):
        checks.check_scores(bad, rs, rc, bound)


def test_selection_rule(score_case):
    q, w, row_seq, keys, ks, scale, rs, rc, bound = score_case
    kw = 100
    sel = oracle.topk_pools(rs, rc, kw)
    checks.check_selection(sel, sel, rs, rc, bound)
    # swap the best selected pool for the worst candidate: far from the cutoff
    bad = sel.copy()
    r = 0
    cand = np.nonzero(rc[r])[0]
    worst = cand[np.argmin(rs[r, cand])]
    best = sel[r][np.argmax(rs[r, sel[r]])]
    row = sorted(set(sel[r]) - {best} | {worst})
    bad[r] = row
    with pytest.raises(AssertionError):
        checks.check_selection(bad, sel, rs, rc, bound)
    # equal scores at the cutoff: either pool may be taken
    rs2 = rs.copy()
    out_pool = next(p for p in cand if p not in set(sel[r]))
    cut_pool = min(sel[r], key=lambda p: rs[r, p])
    rs2[r, out_pool] = rs2[r, cut_pool]
    sel2 = oracle.topk_pools(rs2, rc, kw)
    lo, hi = sorted((int(out_pool), int(cut_pool)))
    assert lo in set(sel2[r]) and hi not in set(sel2[r])       # ties go to the lower pool
    alt = sel2.copy()
    alt[r] = sorted(set(sel2[r]) - {lo} | {hi})
    checks.check_selection(alt, sel2, rs2, rc, bound)

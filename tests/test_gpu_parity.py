"""Parity of the HIP path (through the C ABI) with the CPU oracle, stage by stage.

Each GPU stage gets the same input bytes as the oracle stage it is compared with. Inputs
come from the seeded generators or from the oracle's own previous stage, never from the GPU.

* integer / index work (compact, top-k, expand, selections on exact twins): bit-exact;
* index scores: |gpu - ref| <= 1e-3 |ref| + the f32 error bound of the score (exact twins:
  bit-exact);
* selections on general inputs: differences only among pools within 1e-3 |cutoff| of the
  cutoff score (plus the scores' f32 bounds);
* pooled keys: within one bf16 ulp (+1e-6), exact twins bit-exact;
* sparse MLA: |gpu - ref| <= 2e-2 + 1e-2 |ref| with a bf16 latent, 5e-2 + 1e-2 |ref| fp8,
  and per (row, head) max|d| <= 1e-2 max|ref| and ||d|| <= 1e-2 ||ref||.

The rules themselves are in ``tests/checks.py``.

Full-size workloads run on the GPU exactly as the benchmark launches them; the oracle checks
sampled rows where all rows would take too long.
"""
import numpy as np
import pytest
import torch

import oracle
from dsa_pooled_key_amd import binding as dsa
from tests import checks
from dsa_pooled_key_amd import synth
from dsa_pooled_key_amd.pipeline import DecodeStep, DeviceDecodeInputs, config_for

pytestmark = pytest.mark.gpu

SMALL = ["tiny", "ragged_bf16", "ragged_fp8", "ragged_prefill"]
FULL = ["decode_b8_32k", "decode_b4_256k", "prefill_2048_64k", "fp8_mixed_b32",
        "decode_b8_128k"]
ALL = SMALL + FULL
# The batch-scaling workload (fp8_mixed_b32's recipe at 128 rows): the decode chain's
# launches on it, rows sampled.
SCALE = ["fp8_mixed_b128"]

_CACHE = {}


def setup_module():
    if not torch.cuda.is_available():
        pytest.fail("GPU parity tests need a GPU")
    print(f"\n[gpu] {torch.cuda.get_device_name(0)} libdsa: {dsa.version()}", flush=True)


def case(name, exact=False, peaked=False):
    key = (name, exact, peaked)
    if key not in _CACHE:
        print(f"\n[gpu] generating {name} exact={exact} peaked={peaked}", flush=True)
        di = synth.make_decode_inputs(name, exact=exact, peaked=peaked)
        x = DeviceDecodeInputs.upload(di)
        ids, nv = oracle.compact_pools(di.pool_valid)
        _CACHE[key] = (di, x, ids, nv)
    return _CACHE[key]


def _rows(di, n_small, seed=0):
    Q = di.wl.Q
    if Q <= n_small + 2:
        return np.arange(Q)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, Q - 1), size=n_small, replace=False)
    return np.unique(np.r_[0, mid, Q - 1])


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _oracle_scores(di, ids, nv, rows):
    wl = di.wl
    return oracle.index_scores(di.q[rows], di.w[rows], di.row_seq[rows], di.row_pos[rows],
                               di.keys, ids, nv, kpool=wl.kpool, first_key=wl.first_key,
                               scale=di.scale, key_scales=di.key_scales)


def _bound(di, rows, q=None, w=None, row_seq=None, keys=None, key_scales=None):
    """f32 error bound of the oracle's scores on the given rows."""
    return checks.score_error_bound(di.q[rows] if q is None else q,
                                    di.w[rows] if w is None else w,
                                    di.row_seq[rows] if row_seq is None else row_seq,
                                    di.keys if keys is None else keys,
                                    di.key_scales if keys is None else key_scales, di.scale)


def _check_scores(gs, rs, rc, bound):
    checks.check_scores(gs, rs, rc, bound)


def _check_mla(go, gl, ro, rl, fp8):
    rmax, rl2 = checks.check_mla(go, gl, ro, rl, fp8)
    print(f"[mla] worst max|d|/max|ref| {rmax:.2e}, L2 {rl2:.2e}", flush=True)


# ------------------------------------------------------------------ step 2: compact_pools

@pytest.mark.parametrize("name", ALL)
def test_compact_pools_bit_exact(name):
    di, x, ids, nv = case(name)
    g_ids, g_nv = dsa.compact_pools(x.pool_valid)
    assert np.array_equal(g_nv.cpu().numpy(), nv)
    assert np.array_equal(g_ids.cpu().numpy(), ids)


# ------------------------------------------------------------------ step 3: index_scores

@pytest.mark.parametrize("name", ALL)
def test_index_scores(name):
    di, x, ids, nv = case(name)
    wl = di.wl
    cfg = config_for(wl)
    scores, cand = dsa.index_scores(cfg, x.q, x.w, x.row_seq, x.row_pos, x.keys, _dev(ids),
                                    _dev(nv), first_key=wl.first_key, scale=di.scale,
                                    key_scales=x.key_scales)
    rows = _rows(di, 14)
    rs, rc = _oracle_scores(di, ids, nv, rows)
    gs, gc = scores.cpu().numpy()[rows], cand.cpu().numpy()[rows]
    assert np.array_equal(gc, rc)
    assert np.all(np.isneginf(gs[rc == 0]))
    assert not np.any(np.signbit(gs[rc == 1]) & (gs[rc == 1] == 0))
    _check_scores(gs, rs, rc, _bound(di, rows))


@pytest.mark.parametrize("name", ALL)
def test_index_scores_exact_twin_bit_exact(name):
    di, x, ids, nv = case(name, exact=True)
    wl = di.wl
    cfg = config_for(wl)
    scores, cand = dsa.index_scores(cfg, x.q, x.w, x.row_seq, x.row_pos, x.keys, _dev(ids),
                                    _dev(nv), first_key=wl.first_key, scale=di.scale,
                                    key_scales=x.key_scales)
    rows = _rows(di, 6)
    rs, rc = _oracle_scores(di, ids, nv, rows)
    gs, gc = scores.cpu().numpy()[rows], cand.cpu().numpy()[rows]
    assert np.array_equal(gc, rc)
    assert np.array_equal(gs.view(np.uint32), rs.view(np.uint32))


# ------------------------------------------------------------------ steps 2 and 3 in one launch

def _compact_index(di, x, pool_valid=None, row_seq=None, row_pos=None):
    wl = di.wl
    return dsa.compact_index_scores(
        config_for(wl), x.q, x.w, x.row_seq if row_seq is None else row_seq,
        x.row_pos if row_pos is None else row_pos, x.keys,
        x.pool_valid if pool_valid is None else pool_valid, first_key=wl.first_key,
        scale=di.scale, key_scales=x.key_scales)


@pytest.mark.parametrize("name", ALL + SCALE)
def test_compact_index_scores(name):
    di, x, ids, nv = case(name)
    scores, cand = _compact_index(di, x)
    rows = _rows(di, 14)
    rs, rc = _oracle_scores(di, ids, nv, rows)
    gs, gc = scores.cpu().numpy()[rows], cand.cpu().numpy()[rows]
    assert np.array_equal(gc, rc)
    assert np.all(np.isneginf(gs[rc == 0]))
    assert not np.any(np.signbit(gs[rc == 1]) & (gs[rc == 1] == 0))
    _check_scores(gs, rs, rc, _bound(di, rows))


@pytest.mark.parametrize("name", ALL)
def test_compact_index_scores_exact_twin_bit_exact(name):
    di, x, ids, nv = case(name, exact=True)
    scores, cand = _compact_index(di, x)
    rows = _rows(di, 6)
    rs, rc = _oracle_scores(di, ids, nv, rows)
    gs, gc = scores.cpu().numpy()[rows], cand.cpu().numpy()[rows]
    assert np.array_equal(gc, rc)
    assert np.array_equal(gs.view(np.uint32), rs.view(np.uint32))


@pytest.mark.parametrize("name", ["tiny", "ragged_fp8", "ragged_prefill", "fp8_mixed_b32",
                                  "decode_b4_256k"])
def test_compact_index_scores_equals_the_two_calls(name):
    """Every slot of every row, bit for bit, against compact_pools + index_scores."""
    di, x, _, _ = case(name)
    wl = di.wl
    cfg = config_for(wl)
    ids = torch.empty((wl.B, wl.pools), dtype=torch.int32, device=x.q.device)
    nv = torch.empty((wl.B,), dtype=torch.int32, device=x.q.device)
    dsa.compact_pools(x.pool_valid, ids, nv)
    s2, c2 = dsa.index_scores(cfg, x.q, x.w, x.row_seq, x.row_pos, x.keys, ids, nv,
                              first_key=wl.first_key, scale=di.scale, key_scales=x.key_scales)
    s1, c1 = _compact_index(di, x)
    assert np.array_equal(c1.cpu().numpy(), c2.cpu().numpy())
    assert np.array_equal(s1.cpu().numpy().view(np.uint32), s2.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("name", ["decode_b8_32k", "ragged_fp8"])
def test_compact_index_scores_more_rows_than_threads(name):
    """300 rows over the workload's sequences (rows drawn with replacement, positions redrawn
    below each sequence's length): more rows than a block has threads, so the ranges are not
    reordered, and on decode_b8_32k (300 x 64 ranges) the grid walks them. Every slot equals
    compact_pools + index_scores bit for bit; sampled rows match the oracle."""
    di, x, _, _ = case(name)
    wl = di.wl
    cfg = config_for(wl)
    rng = np.random.default_rng(7)
    R = 300
    src = rng.integers(0, wl.Q, size=R)
    row_seq = di.row_seq[src].astype(np.int32)
    row_pos = (rng.random(R) * di.lengths[row_seq]).astype(np.int32)
    q, w = _dev(di.q[src].view(np.int16)).view(torch.bfloat16), _dev(di.w[src])
    rs_d, rp_d = _dev(row_seq), _dev(row_pos)
    s1, c1 = dsa.compact_index_scores(cfg, q, w, rs_d, rp_d, x.keys, x.pool_valid,
                                      first_key=wl.first_key, scale=di.scale,
                                      key_scales=x.key_scales)
    ids = torch.empty((wl.B, wl.pools), dtype=torch.int32, device=x.q.device)
    nv = torch.empty((wl.B,), dtype=torch.int32, device=x.q.device)
    dsa.compact_pools(x.pool_valid, ids, nv)
    s2, c2 = dsa.index_scores(cfg, q, w, rs_d, rp_d, x.keys, ids, nv, first_key=wl.first_key,
                              scale=di.scale, key_scales=x.key_scales)
    assert np.array_equal(c1.cpu().numpy(), c2.cpu().numpy())
    assert np.array_equal(s1.cpu().numpy().view(np.uint32), s2.cpu().numpy().view(np.uint32))
    rows = np.unique(np.r_[0, rng.choice(R, size=6, replace=False), R - 1])
    ids_o, nv_o = oracle.compact_pools(di.pool_valid)
    rs, rc = oracle.index_scores(di.q[src][rows], di.w[src][rows], row_seq[rows], row_pos[rows],
                                 di.keys, ids_o, nv_o, kpool=wl.kpool, first_key=wl.first_key,
                                 scale=di.scale, key_scales=di.key_scales)
    gs, gc = s1.cpu().numpy()[rows], c1.cpu().numpy()[rows]
    assert np.array_equal(gc, rc)
    _check_scores(gs, rs, rc, _bound(di, rows, q=di.q[src][rows], w=di.w[src][rows],
                                     row_seq=row_seq[rows]))


@pytest.mark.parametrize("name", ["ragged_prefill", "ragged_fp8"])
def test_compact_index_scores_rows_of_one_sequence(name):
    """Many rows over one sequence take the row-blocked scorer (16 rows x 128 pools a block):
    21 rows (a ragged row group) at random positions, some before first_key, one outside the
    batch, against the oracle; the pool count is not a multiple of 128."""
    di, x, _, _ = case(name)
    wl = di.wl
    assert wl.pools % 128 != 0
    rng = np.random.default_rng(11)
    R = 21
    src = rng.integers(0, wl.Q, size=R)
    q, w = di.q[src], di.w[src]
    row_seq = np.zeros(R, np.int32)
    row_seq[5] = -1
    row_pos = rng.integers(0, wl.S, size=R).astype(np.int32)
    row_pos[:3] = [wl.first_key - 1, wl.first_key + wl.kpool // 2, wl.S - 1]
    keys1, pv1 = di.keys[:1], di.pool_valid[:1]
    ks1 = None if di.key_scales is None else di.key_scales[:1]
    ids, nv = oracle.compact_pools(pv1)
    cfg = config_for(wl)
    keys_dev = x.keys[:1].contiguous()
    scores, cand = dsa.compact_index_scores(
        cfg, _dev(q.view(np.int16)).view(torch.bfloat16), _dev(w), _dev(row_seq), _dev(row_pos),
        keys_dev,
        _dev(pv1), first_key=wl.first_key, scale=di.scale,
        key_scales=None if ks1 is None else _dev(ks1))
    gs, gc = scores.cpu().numpy(), cand.cpu().numpy()
    assert not gc[5].any() and np.all(np.isneginf(gs[5]))
    ok = np.array([i for i in range(R) if i != 5])
    rs, rc = oracle.index_scores(q[ok], w[ok], row_seq[ok], row_pos[ok], keys1, ids, nv,
                                 kpool=wl.kpool, first_key=wl.first_key, scale=di.scale,
                                 key_scales=ks1)
    assert np.array_equal(gc[ok], rc)
    assert rc[0].sum() == 0 and rc[2].sum() == nv[0]
    assert np.all(np.isneginf(gs[ok][rc == 0]))
    _check_scores(gs[ok], rs, rc, _bound(di, None, q=q[ok], w=w[ok], row_seq=row_seq[ok],
                                         keys=keys1, key_scales=ks1))


def test_compact_index_scores_edge_rows():
    """Rows outside the batch, a position before first_key, a position in the middle of a pool
    over a sequence whose flags are all nonzero (not only 1), a sequence with no valid pool;
    374 pools, so the last tile of a row is ragged."""
    di, x, _, _ = case("ragged_fp8")
    wl = di.wl
    Q, B, P = wl.Q, wl.B, wl.pools
    assert Q == 5 and list(di.row_seq) == [0, 1, 2, 3, 4] and P % 32 != 0
    row_seq = di.row_seq.copy()
    row_pos = di.row_pos.copy()
    row_seq[0] = -1
    row_seq[1] = B
    row_pos[2] = wl.first_key - 1
    row_pos[3] = wl.first_key + 5 * wl.kpool + wl.kpool // 2
    pv = di.pool_valid.copy()
    pv[3] = np.random.default_rng(7).integers(1, 3, size=P)
    pv[4] = 0
    ids, nv = oracle.compact_pools(pv)
    scores, cand = _compact_index(di, x, pool_valid=_dev(pv), row_seq=_dev(row_seq),
                                  row_pos=_dev(row_pos))
    gs, gc = scores.cpu().numpy(), cand.cpu().numpy()
    # rows 0 and 1 name no sequence of the batch: every slot is a non-candidate
    assert not gc[:2].any() and np.all(np.isneginf(gs[:2]))
    ok = np.arange(2, Q)
    rs, rc = oracle.index_scores(di.q[ok], di.w[ok], row_seq[ok], row_pos[ok], di.keys, ids, nv,
                                 kpool=wl.kpool, first_key=wl.first_key, scale=di.scale,
                                 key_scales=di.key_scales)
    assert np.array_equal(gc[ok], rc)
    assert rc[0].sum() == 0 and rc[1].sum() == 5 and rc[2].sum() == 0
    assert np.all(np.isneginf(gs[ok][rc == 0]))
    _check_scores(gs[ok], rs, rc, _bound(di, ok, row_seq=row_seq[ok]))


# ------------------------------------------------------------------ steps 4 and 5

@pytest.mark.parametrize("name", ALL + SCALE)
def test_topk_and_expand_bit_exact_on_oracle_scores(name):
    di, x, ids, nv = case(name)
    wl = di.wl
    cfg = config_for(wl)
    rows = _rows(di, 14)
    rs, rc = _oracle_scores(di, ids, nv, rows)
    sel_ref = oracle.topk_pools(rs, rc, wl.kw)
    sel = dsa.topk_pools(cfg, _dev(rs), _dev(rc))
    assert np.array_equal(sel.cpu().numpy(), sel_ref)
    tok_ref = oracle.expand_selection(sel_ref, di.row_seq[rows], di.row_pos[rows], di.valid,
                                      kpool=wl.kpool, index_topk=wl.topk,
                                      always_select_tail=wl.tail, first_key=wl.first_key)
    tok = dsa.expand_selection(cfg, _dev(sel_ref), _dev(di.row_seq[rows]),
                               _dev(di.row_pos[rows]), x.valid, S=wl.S, first_key=wl.first_key)
    assert np.array_equal(tok.cpu().numpy(), tok_ref)
    # the fused launch gives both at once
    fsel, ftok = dsa.topk_expand(cfg, _dev(rs), _dev(rc), _dev(di.row_seq[rows]),
                                 _dev(di.row_pos[rows]), x.valid, S=wl.S, first_key=wl.first_key)
    assert np.array_equal(fsel.cpu().numpy(), sel_ref)
    assert np.array_equal(ftok.cpu().numpy(), tok_ref)


@pytest.mark.parametrize("P,kw,seed", [(1, 1, 0), (100, 7, 1), (1024, 512, 2), (1025, 512, 3),
                                       (5000, 300, 4), (16384, 512, 5), (32769, 512, 6),
                                       (65536, 512, 7), (65536, 1, 8), (3000, 3000, 9)])
def test_topk_ties_signs_and_row_lengths(P, kw, seed):
    rng = np.random.default_rng(seed)
    Q = 6
    scores = (rng.integers(-40, 41, (Q, P)) / 8.0).astype(np.float32)   # heavy ties
    scores[1] = 0.0
    scores[1, ::3] = -0.0                                                # signed zeros tie
    scores[2] = rng.standard_normal(P).astype(np.float32) * 1e-30        # tiny magnitudes
    scores[3] = -np.abs(rng.standard_normal(P)).astype(np.float32)       # all negative
    cand = (rng.random((Q, P)) < 0.7).astype(np.uint8)
    cand[4] = 0
    cand[4, : max(1, kw // 2)] = 1                                       # fewer than kw
    cand[5] = 0                                                          # none
    scores[cand == 0] = -np.inf
    cfg = dsa.Config.make(index_heads=32, index_head_dim=128, index_kpool=1, index_topk=kw,
                          heads=32)
    got = dsa.topk_pools(cfg, _dev(scores), _dev(cand)).cpu().numpy()
    ref = oracle.topk_pools(scores, cand, min(kw, P))
    assert np.array_equal(got, ref)
    # fused with expansion (kpool 1: token id = pool id, no tail)
    zeros = _dev(np.zeros(Q, np.int32))
    fsel, ftok = dsa.topk_expand(cfg, _dev(scores), _dev(cand), zeros, zeros,
                                 _dev(np.ones((1, P), np.uint8)), S=P, first_key=0)
    assert np.array_equal(fsel.cpu().numpy(), ref)
    tok_ref = np.full((Q, kw), -1, np.int32)
    tok_ref[:, : ref.shape[1]] = ref
    assert np.array_equal(ftok.cpu().numpy(), tok_ref)


@pytest.mark.parametrize("P,kw", [(16384, 512), (12000, 300)])
def test_topk_more_rows_than_compute_units(P, kw):
    """300 rows of 16 keys a thread, more rows than compute units: the 64-register form that
    puts two blocks on a CU. Rows cycle through heavy ties, signed zeros, tiny magnitudes,
    all-negative scores, fewer candidates than kw, none, and plain normal scores; every row
    bit-exact against the oracle, plain and fused with expansion."""
    rng = np.random.default_rng(11)
    Q = 300
    scores = rng.standard_normal((Q, P)).astype(np.float32)
    cand = (rng.random((Q, P)) < 0.8).astype(np.uint8)
    for r in range(0, Q, 7):
        kind = (r // 7) % 6
        if kind == 0:
            scores[r] = rng.integers(-40, 41, P) / 8.0
        elif kind == 1:
            scores[r] = 0.0
            scores[r, ::3] = -0.0
        elif kind == 2:
            scores[r] = rng.standard_normal(P) * 1e-30
        elif kind == 3:
            scores[r] = -np.abs(rng.standard_normal(P))
        elif kind == 4:
            cand[r] = 0
            cand[r, : kw // 2] = 1
        else:
            cand[r] = 0
    scores[cand == 0] = -np.inf
    cfg = dsa.Config.make(index_heads=32, index_head_dim=128, index_kpool=1, index_topk=kw,
                          heads=32)
    ref = oracle.topk_pools(scores, cand, kw)
    got = dsa.topk_pools(cfg, _dev(scores), _dev(cand)).cpu().numpy()
    assert np.array_equal(got, ref)
    zeros = _dev(np.zeros(Q, np.int32))
    fsel, ftok = dsa.topk_expand(cfg, _dev(scores), _dev(cand), zeros, zeros,
                                 _dev(np.ones((1, P), np.uint8)), S=P, first_key=0)
    assert np.array_equal(fsel.cpu().numpy(), ref)
    assert np.array_equal(ftok.cpu().numpy(), ref)


@pytest.mark.parametrize("P,kw,seed", [(8192, 512, 40), (16384, 512, 41), (16384, 100, 42),
                                       (32768, 512, 43), (32768, 2048, 44)])
def test_topk_rows_of_many_candidates_a_thread(P, kw, seed):
    """One block a row with at least 8 pools a thread and four times kw candidates or more:
    rows whose candidates sit in fewer than kw threads, ascending and descending scores, ties
    at the cutoff across many threads, one huge outlier, sparse candidates and plain normal
    scores."""
    rng = np.random.default_rng(seed)
    Q = 8
    scores = rng.standard_normal((Q, P)).astype(np.float32)
    cand = np.ones((Q, P), np.uint8)
    cand[0] = 0
    cand[0, : 4 * kw + 16] = 1                                         # few threads hold them
    scores[1] = np.linspace(-3.0, 3.0, P, dtype=np.float32)            # ascending
    scores[2] = np.linspace(3.0, -3.0, P, dtype=np.float32)            # descending
    scores[3] = (rng.integers(0, 4, P) / 2.0).astype(np.float32)       # ties at the cutoff
    scores[4, rng.integers(0, P)] = 1.0e30                             # one outlier
    scores[5] = np.where(rng.random(P) < 0.5, 2.0, scores[5]).astype(np.float32)
    cand[6] = (rng.random(P) < 0.3).astype(np.uint8)                   # sparse candidates
    scores[cand == 0] = -np.inf
    cfg = dsa.Config.make(index_heads=32, index_head_dim=128, index_kpool=1, index_topk=kw,
                          heads=32)
    got = dsa.topk_pools(cfg, _dev(scores), _dev(cand), ws=False).cpu().numpy()
    ref = oracle.topk_pools(scores, cand, min(kw, P))
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("P,kw,seed", [(16385, 512, 20), (24577, 512, 21), (32768, 512, 22),
                                       (65536, 512, 23), (40000, 100, 24), (32768, 2048, 25)])
def test_topk_two_stage_equals_one_block(P, kw, seed):
    """The two-launch selection (segments' best, then the row's best among them) against the
    one-block selection and the oracle, on rows with heavy ties across segment boundaries,
    equal scores only in some segments, and rows with fewer candidates than kw."""
    rng = np.random.default_rng(seed)
    Q = 5
    scores = (rng.integers(-6, 7, (Q, P)) / 4.0).astype(np.float32)
    scores[1] = rng.standard_normal(P).astype(np.float32)
    scores[2, : P // 2] = 1.0                                  # one value over several segments
    cand = (rng.random((Q, P)) < 0.8).astype(np.uint8)
    cand[3] = 0
    cand[3, rng.choice(P, kw // 2, replace=False)] = 1         # fewer than kw
    cand[4] = 0
    scores[cand == 0] = -np.inf
    cfg = dsa.Config.make(index_heads=32, index_head_dim=128, index_kpool=1, index_topk=kw,
                          heads=32)
    assert dsa.topk_workspace(cfg, Q, P) > 0
    two = dsa.topk_pools(cfg, _dev(scores), _dev(cand)).cpu().numpy()
    one = dsa.topk_pools(cfg, _dev(scores), _dev(cand), ws=False).cpu().numpy()
    ref = oracle.topk_pools(scores, cand, min(kw, P))
    assert np.array_equal(two, ref) and np.array_equal(one, ref)
    zeros = _dev(np.zeros(Q, np.int32))
    fsel, ftok = dsa.topk_expand(cfg, _dev(scores), _dev(cand), zeros, zeros,
                                 _dev(np.ones((1, P), np.uint8)), S=P, first_key=0)
    assert np.array_equal(fsel.cpu().numpy(), ref)


# ------------------------------------------------------------------ step 6: sparse MLA

@pytest.mark.parametrize("name", ALL + SCALE)
def test_sparse_mla_decode(name):
    di, x, _, _ = case(name)
    wl = di.wl
    cfg = config_for(wl)
    tok = synth.draw_token_ids(di)
    out, lse = dsa.sparse_mla_decode(cfg, x.q_abs, _dev(tok), x.row_seq, x.kv, B=wl.B,
                                     sm_scale=di.sm_scale, S=wl.S, kv_scales=x.kv_scales,
                                     block_table=x.block_table)
    rows = _rows(di, 64)
    ro, rl = oracle.sparse_mla(di.q_abs[rows], tok[rows], di.row_seq[rows], di.kv,
                               sm_scale=di.sm_scale, S=wl.S, kv_scales=di.kv_scales,
                               block_table=di.block_table)
    _check_mla(out.cpu().numpy()[rows], lse.cpu().numpy()[rows], ro, rl, wl.kv_fp8)


@pytest.mark.parametrize("name", ["ragged_fp8", "decode_b8_32k", "fp8_mixed_b32",
                                  "decode_b8_128k"])
def test_sparse_mla_decode_peaked(name):
    """q_abs drawn so that the logits have standard deviation 3 (synth.PEAKED_QABS_STD): the
    softmax puts most of a row's weight on a few dozen of its thousands of tokens, so the
    output is large and the products, the split partials and their merge decide it."""
    di, x, _, _ = case(name)
    wl = di.wl
    cfg = config_for(wl)
    q_abs = synth.peaked_q_abs(name)
    tok = synth.draw_token_ids(di)
    out, lse = dsa.sparse_mla_decode(cfg, _dev(q_abs.view(np.int16)).view(torch.bfloat16),
                                     _dev(tok), x.row_seq, x.kv, B=wl.B, sm_scale=di.sm_scale,
                                     S=wl.S, kv_scales=x.kv_scales, block_table=x.block_table)
    rows = _rows(di, 16)
    ro, rl = oracle.sparse_mla(q_abs[rows], tok[rows], di.row_seq[rows], di.kv,
                               sm_scale=di.sm_scale, S=wl.S, kv_scales=di.kv_scales,
                               block_table=di.block_table)
    live = ~np.isneginf(rl)
    assert np.abs(ro).max(-1)[live].min() > 0.1     # far from the uniform-softmax regime
    _check_mla(out.cpu().numpy()[rows], lse.cpu().numpy()[rows], ro, rl, wl.kv_fp8)


@pytest.mark.parametrize("name,n_rows", [("ragged_bf16", 66), ("ragged_fp8", 181)])
def test_sparse_mla_paired_splits(name, n_rows):
    """Enough rows that two splits of a row share one block and merge in LDS (bf16: two head
    groups, 4 splits; fp8 paged: 3 splits, so the last block's second split is empty). Rows 0-3
    are emptied so that either split of a pair, both or neither hold tokens."""
    di, x, _, _ = case(name)
    wl = di.wl
    cfg = config_for(wl)
    rng = np.random.default_rng(11)
    k = (n_rows + wl.Q - 1) // wl.Q
    q = np.tile(di.q_abs, (k, 1, 1))[:n_rows]
    rs = np.tile(di.row_seq, k)[:n_rows].astype(np.int32)
    tok = np.tile(synth.draw_token_ids(di), (k, 1))[:n_rows]
    tok = np.take_along_axis(tok, rng.permuted(np.tile(np.arange(tok.shape[1]), (n_rows, 1)), axis=1), 1)
    W = tok.shape[1]
    tok[0] = -1                # no tokens at all
    tok[1, 64:] = -1           # only the first split
    tok[2, :64] = -1           # the second split only
    tok[2, 128:] = -1
    tok[3, :128] = -1          # only the splits from slot 128 on
    tok = np.ascontiguousarray(tok)
    assert W > 128
    qd = torch.from_numpy(np.ascontiguousarray(q).view(np.int16)).cuda().view(torch.bfloat16)
    out, lse = dsa.sparse_mla_decode(cfg, qd, _dev(tok), _dev(rs), x.kv, B=wl.B,
                                     sm_scale=di.sm_scale, S=wl.S, kv_scales=x.kv_scales,
                                     block_table=x.block_table)
    ro, rl = oracle.sparse_mla(q, tok, rs, di.kv, sm_scale=di.sm_scale, S=wl.S,
                               kv_scales=di.kv_scales, block_table=di.block_table)
    _check_mla(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, wl.kv_fp8)
    assert np.all(np.isneginf(lse.cpu().numpy()[0]))


@pytest.mark.parametrize("n_splits", list(range(2, 17)))
def test_sparse_mla_every_split_count(n_splits):
    """Rows of 64 * n - 13 token slots are cut into n splits of 64 (two rows, one head group),
    so the merge of the split partials runs with every split count it is built for (2..16);
    against the oracle."""
    S, H, Q = 2000, 32, 2
    W = 64 * n_splits - 13
    rng = np.random.default_rng(60 + n_splits)
    kv = synth.bf16_bits(rng.normal(0.0, 0.5, (S, 512)).astype(np.float32))
    q = synth.bf16_bits(rng.normal(0.0, 1.0, (Q, H, 512)).astype(np.float32))
    tok = rng.integers(0, S, (Q, W)).astype(np.int32)
    tok[rng.random(tok.shape) < 0.05] = -1
    tok[1, 64:128] = -1                      # one split of row 1 without tokens
    rs = np.zeros(Q, np.int32)
    cfg = dsa.Config.make(index_heads=32, index_head_dim=128, index_kpool=1, index_topk=W, heads=H)
    assert dsa.sparse_mla_workspace(cfg, Q, W) > 0
    kv_d = torch.from_numpy(kv.view(np.int16)).cuda().view(torch.bfloat16)
    qd = torch.from_numpy(q.view(np.int16)).cuda().view(torch.bfloat16)
    sm = 1.0 / np.sqrt(576.0)
    out, lse = dsa.sparse_mla_decode(cfg, qd, _dev(tok), _dev(rs), kv_d, B=1, sm_scale=sm, S=S)
    ro, rl = oracle.sparse_mla(q, tok, rs, kv, sm_scale=sm, S=S)
    _check_mla(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, False)


@pytest.mark.parametrize("Q,fp8", [(1, False), (64, False), (64, True)])
def test_sparse_mla_widest_selection(Q, fp8):
    """The widest selection the boundary takes (32,768 token slots: 16 splits of 2,048, the
    most the combine merges), on one row (16 one-team splits) and on 64 rows (1,024 teams, so
    two 2,048-slot splits share each block); random tokens of one 40,000-token sequence with
    scattered -1 slots; the last row against the oracle."""
    S, W, H = 40000, 32768, 32
    rng = np.random.default_rng(31 + Q + fp8)
    kvf = rng.normal(0.0, 0.5, (S, 512)).astype(np.float32)
    scales = None
    if fp8:
        kv, scales = synth.e4m3_quantize_rows(kvf)
        kv_d = torch.from_numpy(kv).cuda()
        sc_d = _dev(scales)
    else:
        kv = synth.bf16_bits(kvf)
        kv_d = torch.from_numpy(kv.view(np.int16)).cuda().view(torch.bfloat16)
        sc_d = None
    q = synth.bf16_bits(rng.normal(0.0, 1.0, (Q, H, 512)).astype(np.float32))
    tok = np.stack([rng.permutation(S)[:W] for _ in range(Q)]).astype(np.int32)
    tok[rng.random(tok.shape) < 0.01] = -1
    rs = np.zeros(Q, np.int32)
    cfg = dsa.Config.make(index_heads=32, index_head_dim=128, index_kpool=4, index_topk=W, heads=H)
    qd = torch.from_numpy(q.view(np.int16)).cuda().view(torch.bfloat16)
    sm = 1.0 / np.sqrt(576.0)
    out, lse = dsa.sparse_mla_decode(cfg, qd, _dev(tok), _dev(rs), kv_d, B=1, sm_scale=sm, S=S,
                                     kv_scales=sc_d)
    rows = np.array([Q - 1])
    ro, rl = oracle.sparse_mla(q[rows], tok[rows], rs[rows], kv, sm_scale=sm, S=S,
                               kv_scales=scales)
    _check_mla(out.cpu().numpy()[rows], lse.cpu().numpy()[rows], ro, rl, fp8)


def test_sparse_mla_repeatable_paging_invariant_and_masks_bad_ids():
    di, x, _, _ = case("ragged_bf16")
    wl = di.wl
    cfg = config_for(wl)
    tok = synth.draw_token_ids(di)
    kw = dict(B=wl.B, sm_scale=di.sm_scale, S=wl.S)
    o1, l1 = dsa.sparse_mla_decode(cfg, x.q_abs, _dev(tok), x.row_seq, x.kv, **kw)
    o2, l2 = dsa.sparse_mla_decode(cfg, x.q_abs, _dev(tok), x.row_seq, x.kv, **kw)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # the same rows behind a shuffled 64-token block table: identical bits
    bs = 64
    nb = (wl.S + bs - 1) // bs
    rng = np.random.default_rng(3)
    perm = rng.permutation(wl.B * nb).astype(np.int32)
    table = perm.reshape(wl.B, nb)
    paged = np.zeros((wl.B * nb * bs, 512), np.uint16)
    for b in range(wl.B):
        for j in range(nb):
            n = min(bs, wl.S - j * bs)
            paged[table[b, j] * bs: table[b, j] * bs + n] = di.kv[b * wl.S + j * bs: b * wl.S + j * bs + n]
    kvp = torch.from_numpy(paged.view(np.int16)).cuda().view(torch.bfloat16)
    o3, l3 = dsa.sparse_mla_decode(cfg, x.q_abs, _dev(tok), x.row_seq, kvp, B=wl.B,
                                   sm_scale=di.sm_scale, S=wl.S, block_table=_dev(table))
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    # the same table padded with unmapped columns past what the kernel stages in LDS (the
    # lookups then go to global memory): identical bits
    wide = np.full((wl.B, 9000), -1, np.int32)
    wide[:, :nb] = table
    o3w, l3w = dsa.sparse_mla_decode(cfg, x.q_abs, _dev(tok), x.row_seq, kvp, B=wl.B,
                                     sm_scale=di.sm_scale, S=wl.S, block_table=_dev(wide))
    assert torch.equal(o1, o3w) and torch.equal(l1, l3w)
    # a page size that is not a power of two: identical bits
    bs3 = 48
    nb3 = (wl.S + bs3 - 1) // bs3
    table3 = rng.permutation(wl.B * nb3).astype(np.int32).reshape(wl.B, nb3)
    paged3 = np.zeros((wl.B * nb3 * bs3, 512), np.uint16)
    for b in range(wl.B):
        for j in range(nb3):
            n = min(bs3, wl.S - j * bs3)
            paged3[table3[b, j] * bs3: table3[b, j] * bs3 + n] = \
                di.kv[b * wl.S + j * bs3: b * wl.S + j * bs3 + n]
    kvp3 = torch.from_numpy(paged3.view(np.int16)).cuda().view(torch.bfloat16)
    o3p, l3p = dsa.sparse_mla_decode(cfg, x.q_abs, _dev(tok), x.row_seq, kvp3, B=wl.B,
                                     sm_scale=di.sm_scale, S=wl.S, block_table=_dev(table3),
                                     block_size=bs3)
    assert torch.equal(o1, o3p) and torch.equal(l1, l3p)
    # ids past the sequence, negative ids and unmapped blocks are skipped like -1
    bad = tok.copy()
    bad[0, 5] = wl.S + 10
    bad[1, 7] = -5
    table2 = table.copy()
    blk = int(tok[2, 3]) // bs
    table2[int(di.row_seq[2]), blk] = -1
    clean = bad.copy()
    clean[clean >= wl.S] = -1
    clean[clean < 0] = -1
    clean[2][(tok[2] >= 0) & (tok[2] // bs == blk)] = -1
    o4, l4 = dsa.sparse_mla_decode(cfg, x.q_abs, _dev(bad), x.row_seq, kvp, B=wl.B,
                                   sm_scale=di.sm_scale, S=wl.S, block_table=_dev(table2))
    ro, rl = oracle.sparse_mla(di.q_abs, clean, di.row_seq, di.kv, sm_scale=di.sm_scale, S=wl.S)
    _check_mla(o4.cpu().numpy(), l4.cpu().numpy(), ro, rl, False)
    # empty rows
    empty = np.full_like(tok, -1)
    o5, l5 = dsa.sparse_mla_decode(cfg, x.q_abs, _dev(empty), x.row_seq, x.kv, **kw)
    assert torch.all(o5 == 0) and torch.all(torch.isneginf(l5))


# ------------------------------------------------------------------ step 1: kpool_compress

KPOOL_BATCH = {"fp8_mixed_b32": 6, "decode_b4_256k": 2, "decode_b8_128k": 2}


@pytest.mark.parametrize("exact", [False, True])
@pytest.mark.parametrize("name", ALL)
def test_kpool_compress(name, exact):
    ki = synth.make_kpool_inputs(name, exact=exact, batch=KPOOL_BATCH.get(name))
    wl = ki.wl
    cfg = config_for(wl)
    k = _dev(ki.k.view(np.int16)).view(torch.bfloat16)
    g = _dev(ki.gate.view(np.int16)).view(torch.bfloat16)
    pk, pv = dsa.kpool_compress(cfg, k, g, _dev(ki.ape), _dev(ki.valid), wl.first_key)
    rk, rv = oracle.kpool_compress(ki.k, ki.gate, ki.ape, ki.valid, wl.kpool, wl.first_key)
    assert np.array_equal(pv.cpu().numpy(), rv)
    got = pk.view(torch.int16).cpu().numpy().view(np.uint16)
    a = synth.bf16_to_f32(got).astype(np.float64)
    b = synth.bf16_to_f32(rk).astype(np.float64)
    if exact:
        # Compared by value: with one-hot weights the exact pooled key is the hot slot's key
        # plus about 1e-56 times the others, which the f64 oracle rounds to -0 when the hot key
        # is 0 and the GPU, whose exp(-128) underflows to 0 in f32, writes as +0.
        assert np.array_equal(a, b)
        return
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(b), 2.0 ** -126))) - 7)
    bad = np.abs(a - b) > ulp + 1e-6
    assert not bad.any(), (np.argwhere(bad)[:4], a[bad][:4], b[bad][:4])


@pytest.mark.parametrize("exact", [False, True])
@pytest.mark.parametrize("name", ALL)
def test_kpool_compress_fp8(name, exact):
    """fp8 pooled keys: the GPU's own bf16 pooled key (the bf16 launch, same arithmetic)
    quantized by the oracle's quantizer gives the fp8 launch's codes and scales bit for bit;
    on the exact twins the codes equal the oracle's whole fp8 pooling by value (+-0 alike)."""
    ki = synth.make_kpool_inputs(name, exact=exact, batch=KPOOL_BATCH.get(name))
    wl = ki.wl
    cfg = config_for(wl)
    k = _dev(ki.k.view(np.int16)).view(torch.bfloat16)
    g = _dev(ki.gate.view(np.int16)).view(torch.bfloat16)
    ape, valid = _dev(ki.ape), _dev(ki.valid)
    pk, pv = dsa.kpool_compress(cfg, k, g, ape, valid, wl.first_key)
    codes, sc, pv8 = dsa.kpool_compress_fp8(cfg, k, g, ape, valid, wl.first_key)
    assert torch.equal(pv, pv8)
    gvals = synth.bf16_to_f32(pk.view(torch.int16).cpu().numpy().view(np.uint16))
    rc, rs = oracle.quantize_rows(gvals)
    assert np.array_equal(sc.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)
    if exact:
        oc, osc, opv = oracle.kpool_compress_fp8(ki.k, ki.gate, ki.ape, ki.valid, wl.kpool,
                                                 wl.first_key)
        assert np.array_equal(pv8.cpu().numpy(), opv)
        assert np.array_equal(sc.cpu().numpy(), osc)
        dec = np.vectorize(oracle.e4m3_value, otypes=[np.float64])
        got = codes.cpu().numpy()
        lut = dec(np.arange(256, dtype=np.uint8))
        assert np.array_equal(lut[got], lut[oc])


def _quant_rows_case(n, rng):
    rows = [rng.standard_normal(n) * 0.5,
            np.zeros(n),
            np.where(np.arange(n) == 3, -2.75, 0.0),
            rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n)),     # wide range
            rng.standard_normal(n) * 1e-3]
    # s = 1 (amax 448): every other value a midpoint between two e4m3 values (ties to even)
    vals = np.array([oracle.e4m3_value(c) for c in range(0x7f)])
    mids = (vals[:-1] + vals[1:]) / 2
    t = rng.choice(mids, n) * rng.choice([-1.0, 1.0], n)
    t[0] = 448.0
    rows.append(t)
    neg0 = np.full(n, -0.0)
    neg0[1] = 1.0
    rows.append(neg0)
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("n", [8, 72, 512, 4096])
def test_quantize_rows_fp8_bit_exact(n):
    """Latent-row quantizer, bf16 and f32 sources: codes and scales bit-exact with the
    oracle, on random rows, zero rows, a single nonzero, a 2^+-30 dynamic range, values in
    the subnormal range, exact midpoints (ties to even) and negative zeros; also 1200 rows of
    512 (the latent width) drawn like the latent cache."""
    rng = np.random.default_rng(n)
    x = _quant_rows_case(n, rng)
    if n == 512:
        x = np.concatenate([x, (rng.standard_normal((1200, n)) * 0.5).astype(np.float32)])
    for src in (x, synth.bf16_to_f32(synth.bf16_bits(x))):
        rc, rs = oracle.quantize_rows(src)
        for dt in ((torch.float32,) if src is x else (torch.bfloat16, torch.float32)):
            t = torch.from_numpy(src).cuda().to(dt)
            codes, sc = dsa.quantize_rows_fp8(t)
            assert np.array_equal(sc.cpu().numpy(), rs), dt
            got = codes.cpu().numpy()
            bad = np.argwhere(got != rc)
            assert bad.size == 0, (dt, bad[:5], got[tuple(bad[0])], rc[tuple(bad[0])],
                                   src[tuple(bad[0])] / rs[bad[0][0]])


# ------------------------------------------------------------------ dense masked cross-check

@pytest.mark.parametrize("name", ALL)
def test_topk_to_mask_bit_exact(name):
    di, x, _, _ = case(name)
    wl = di.wl
    tok = synth.draw_token_ids(di)
    rows = _rows(di, 30)
    tok = np.ascontiguousarray(tok[rows])
    tok[0, :5] = [wl.S, wl.S + 7, -3, tok[0, 5], tok[0, 5]]   # out of range and duplicates
    m = dsa.topk_to_mask(_dev(tok), wl.S)
    assert np.array_equal(m.cpu().numpy(), oracle.topk_to_mask(tok, wl.S))


MASKED = ["tiny", "ragged_bf16", "ragged_fp8", "ragged_prefill", "decode_b8_32k"]


@pytest.mark.parametrize("name", MASKED)
def test_masked_attn_against_oracle_and_sparse_decode(name):
    """The dense masked attention against the oracle's (sampled rows), and the cross-check
    itself: sparse decode over token ids and dense attention over their mask agree within the
    decode tolerance on every row."""
    di, x, _, _ = case(name)
    wl = di.wl
    cfg = config_for(wl)
    tok = synth.draw_token_ids(di)
    mask = dsa.topk_to_mask(_dev(tok), wl.S)
    kw = dict(sm_scale=di.sm_scale, kv_scales=x.kv_scales, block_table=x.block_table)
    mo, ml = dsa.mla_masked_attn(cfg, x.q_abs, mask, x.row_seq, x.kv, B=wl.B, **kw)
    rows = _rows(di, 6)
    ro, rl = oracle.masked_attn(di.q_abs[rows], oracle.topk_to_mask(tok[rows], wl.S),
                                di.row_seq[rows], di.kv, sm_scale=di.sm_scale,
                                kv_scales=di.kv_scales, block_table=di.block_table)
    _check_mla(mo.cpu().numpy()[rows], ml.cpu().numpy()[rows], ro, rl, wl.kv_fp8)
    so, sl = dsa.sparse_mla_decode(cfg, x.q_abs, _dev(tok), x.row_seq, x.kv, B=wl.B, S=wl.S, **kw)
    _check_mla(so.cpu().numpy(), sl.cpu().numpy(), mo.cpu().numpy().astype(np.float64),
               ml.cpu().numpy().astype(np.float64), wl.kv_fp8)


def test_masked_attn_empty_rows_and_the_key_limit():
    di, x, _, _ = case("ragged_bf16")
    wl = di.wl
    cfg = config_for(wl)
    mask = torch.zeros((wl.Q, wl.S), dtype=torch.uint8, device="cuda")
    o, l = dsa.mla_masked_attn(cfg, x.q_abs, mask, x.row_seq, x.kv, B=wl.B, sm_scale=di.sm_scale)
    assert torch.all(o == 0) and torch.all(torch.isneginf(l))
    big = torch.zeros((1, 32769), dtype=torch.uint8, device="cuda")
    with pytest.raises(dsa.DsaError):
        dsa.mla_masked_attn(cfg, x.q_abs[:1].contiguous(), big, x.row_seq[:1].contiguous(), x.kv,
                            B=wl.B, sm_scale=di.sm_scale)


# ------------------------------------------------------------------ decode-time upkeep

def _bf(a):
    return _dev(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("D", [32, 64, 128])
def test_k_norm(D):
    """LayerNorm with a bias, in place: within one bf16 ulp of the oracle (f32 against
    double arithmetic); bit-exact on rows whose mean, variance and square root are exact
    (halves at c + a and c - a, a a power of two, eps 0)."""
    rng = np.random.default_rng(D)
    rows = 777
    x = synth.bf16_bits((rng.standard_normal((rows, D)) * rng.uniform(0.1, 4, (rows, 1))
                         + rng.standard_normal((rows, 1)) * 3).astype(np.float32))
    w = synth.bf16_bits((1 + 0.3 * rng.standard_normal(D)).astype(np.float32))
    b = synth.bf16_bits((0.2 * rng.standard_normal(D)).astype(np.float32))
    xt = _bf(x)
    dsa.k_norm(xt, _bf(w), _bf(b), 1e-5)
    ref = synth.bf16_to_f32(oracle.layer_norm(x, w, b, 1e-5)).astype(np.float64)
    got = synth.bf16_to_f32(_bits(xt)).astype(np.float64)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    bad = np.abs(got - ref) > ulp + 1e-7
    assert not bad.any(), (np.argwhere(bad)[:4], got[bad][:4], ref[bad][:4])
    # exact rows
    a = np.exp2(rng.integers(-3, 4, (64, 1)))
    c = rng.integers(-16, 17, (64, 1)) / 4.0
    sign = np.where(rng.permuted(np.tile(np.arange(D) % 2, (64, 1)), axis=1) == 0, -1.0, 1.0)
    xe = synth.bf16_bits((c + a * sign).astype(np.float32))
    we = synth.bf16_bits((rng.integers(-8, 9, D) / 4.0).astype(np.float32))
    be = synth.bf16_bits((rng.integers(-8, 9, D) / 8.0).astype(np.float32))
    xt = _bf(xe)
    dsa.k_norm(xt, _bf(we), _bf(be), 0.0)
    assert np.array_equal(_bits(xt), oracle.layer_norm(xe, we, be, 0.0))


def test_indexer_store_and_write_geom():
    rng = np.random.default_rng(60)
    B, S, D = 6, 50, 128
    kc = rng.integers(0, 65535, (B, S, D)).astype(np.uint16) & 0x7f7f
    gc = rng.integers(0, 65535, (B, S, D)).astype(np.uint16) & 0x7f7f
    valid = (rng.random((B, S)) > 0.5).astype(np.uint8)
    kr = rng.integers(0, 65535, (B, D)).astype(np.uint16) & 0x7f7f
    gr = rng.integers(0, 65535, (B, D)).astype(np.uint16) & 0x7f7f
    pos = np.array([0, 49, 50, -1, 17, 17], np.int32)
    tk, tg, tv = _bf(kc), _bf(gc), _dev(valid)
    dsa.indexer_store(_dev(pos), _bf(kr), _bf(gr), tk, tg, tv)
    rk, rg, rv = oracle.indexer_store(pos, kr, gr, kc, gc, valid)
    assert np.array_equal(_bits(tk), rk) and np.array_equal(_bits(tg), rg)
    assert np.array_equal(tv.cpu().numpy(), rv)
    lens = np.array([1, 131072, 4096, 0, 77, 5000], np.int32)
    rs, rp = dsa.write_geom(_dev(lens))
    ors, orp = oracle.write_geom(lens)
    assert np.array_equal(rs.cpu().numpy(), ors) and np.array_equal(rp.cpu().numpy(), orp)


@pytest.mark.parametrize("kp,f,fp8", [(4, 0, False), (8, 5, True), (3, 2, False), (8, 0, True)])
def test_pool_append_token_by_token_equals_batch(kp, f, fp8):
    """A cache filled one token per step (indexer_store, then pool_append) ends with the pool
    keys, validity and compacted ids of the batch calls (the GPU's own batch pooling, bit for
    bit; the oracle's compaction, bit for bit; the oracle's keys within one bf16 ulp); a
    repeated append changes nothing."""
    rng = np.random.default_rng(61 + kp)
    B, S, D = 3, 70, 128
    cfg = dsa.Config.make(index_heads=32, index_head_dim=D, index_kpool=kp, index_topk=8 * kp,
                          heads=32)
    k = synth.bf16_bits(rng.standard_normal((B, S, D)).astype(np.float32))
    gate = synth.bf16_bits(rng.standard_normal((B, S, D)).astype(np.float32))
    ape = rng.standard_normal((kp, D)).astype(np.float32)
    fv = (rng.random((B, S)) > 0.08).astype(np.uint8)
    P = oracle.num_pools(S, f, kp)
    kc = torch.zeros((B, S, D), dtype=torch.bfloat16, device="cuda")
    gc = torch.zeros_like(kc)
    vc = torch.zeros((B, S), dtype=torch.uint8, device="cuda")
    pk = torch.zeros((B, P, D), dtype=torch.uint8 if fp8 else torch.bfloat16, device="cuda")
    sc = torch.zeros((B, P), dtype=torch.float32, device="cuda") if fp8 else None
    pv = torch.zeros((B, P), dtype=torch.uint8, device="cuda")
    ids = torch.full((B, P), -1, dtype=torch.int32, device="cuda")
    nv = torch.zeros((B,), dtype=torch.int32, device="cuda")
    ta, kt, gt, fvt = _dev(ape), _bf(k), _bf(gate), _dev(fv)
    for t in range(S):
        pos = torch.full((B,), t, dtype=torch.int32, device="cuda")
        dsa.indexer_store(pos, kt[:, t].contiguous(), gt[:, t].contiguous(), kc, gc, vc)
        vc[:, t] = fvt[:, t]
        for _ in range(2):
            dsa.pool_append(cfg, pos, kc, gc, ta, vc, pk, pv, ids, nv, first_key=f,
                            pool_key_scales=sc)
    torch.cuda.synchronize()
    if fp8:
        bk, bsc, bpv = dsa.kpool_compress_fp8(cfg, kt, gt, ta, fvt, f)
        assert torch.equal(sc, bsc)
    else:
        bk, bpv = dsa.kpool_compress(cfg, kt, gt, ta, fvt, f)
    assert torch.equal(pk.view(torch.uint8), bk.view(torch.uint8)) and torch.equal(pv, bpv)
    rk, rv = oracle.kpool_compress(k, gate, ape, fv, kp, f)
    rids, rnv = oracle.compact_pools(rv)
    assert np.array_equal(pv.cpu().numpy(), rv)
    assert np.array_equal(ids.cpu().numpy(), rids) and np.array_equal(nv.cpu().numpy(), rnv)
    if not fp8:
        a = synth.bf16_to_f32(_bits(pk)).astype(np.float64)
        r = synth.bf16_to_f32(rk).astype(np.float64)
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(r), 2.0 ** -126))) - 7)
        assert np.all(np.abs(a - r) <= ulp + 1e-6)


@pytest.mark.parametrize("name", ["ragged_fp8", "ragged_bf16", "decode_b8_32k"])
def test_pool_append_one_decode_step_against_the_oracle(name):
    """One decode step on a workload's token cache, each sequence at its own position (some
    completing a pool, one inside a pool, one past the cache): keys, validity and ids as the
    oracle's append of the same step."""
    ki = synth.make_kpool_inputs(name, batch=KPOOL_BATCH.get(name))
    wl = ki.wl
    cfg = config_for(wl)
    B, S, D = ki.k.shape
    f, kp = wl.first_key, wl.kpool
    rng = np.random.default_rng(62)
    pos = rng.integers(f + kp, S, B).astype(np.int32)
    pos = f + ((pos - f) // kp) * kp + kp - 1                      # each completes a pool
    pos[-1] = S + 3
    if B > 2:
        pos[-2] -= 1                                               # inside a pool
    rk, rv = oracle.kpool_compress(ki.k, ki.gate, ki.ape, ki.valid, kp, f)
    before = rv.copy()
    done = [b for b in range(B) if 0 <= pos[b] < S and (pos[b] - f + 1) % kp == 0]
    for b in done:       # the pool this step completes is not there yet
        before[b, (pos[b] - f + 1) // kp - 1:] = 0
    ids0, nv0 = oracle.compact_pools(before)
    keys0 = np.zeros_like(rk)
    ok_k, ok_v, ok_ids, ok_nv = oracle.pool_append(pos, ki.k, ki.gate, ki.ape, ki.valid, keys0,
                                                   before, ids0, nv0, kpool=kp, first_key=f)
    gk, pv, ids, nv = _bf(keys0), _dev(before), _dev(ids0), _dev(nv0)
    dsa.pool_append(cfg, _dev(pos), _bf(ki.k), _bf(ki.gate), _dev(ki.ape), _dev(ki.valid), gk, pv,
                    ids, nv, first_key=f)
    assert np.array_equal(pv.cpu().numpy(), ok_v)
    assert np.array_equal(ids.cpu().numpy(), ok_ids) and np.array_equal(nv.cpu().numpy(), ok_nv)
    a = synth.bf16_to_f32(_bits(gk)).astype(np.float64)
    r = synth.bf16_to_f32(ok_k).astype(np.float64)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(r), 2.0 ** -126))) - 7)
    assert np.all(np.abs(a - r) <= ulp + 1e-6)
    assert len(done) >= 1 and (nv.cpu().numpy() - nv0).sum() == sum(
        int(rv[b, (pos[b] - f + 1) // kp - 1]) for b in done)


# ------------------------------------------------------------------ chains

def _oracle_select(di, ids, nv, rows):
    wl = di.wl
    rs, rc = _oracle_scores(di, ids, nv, rows)
    sel = oracle.topk_pools(rs, rc, wl.kw)
    tok = oracle.expand_selection(sel, di.row_seq[rows], di.row_pos[rows], di.valid,
                                  kpool=wl.kpool, index_topk=wl.topk,
                                  always_select_tail=wl.tail, first_key=wl.first_key)
    return rs, rc, sel, tok


@pytest.mark.parametrize("name", ALL)
def test_selection_chain_exact_twin_bit_exact(name):
    di, x, ids, nv = case(name, exact=True)
    step = DecodeStep(di.wl, x, di.scale, di.sm_scale)
    step.select()
    rows = _rows(di, 6)
    _, _, sel, tok = _oracle_select(di, ids, nv, rows)
    assert np.array_equal(step.sel.cpu().numpy()[rows], sel)
    assert np.array_equal(step.token_ids.cpu().numpy()[rows], tok)


@pytest.mark.parametrize("name", ["ragged_fp8", "fp8_mixed_b32", "decode_b4_256k"])
def test_fused_and_separate_selection_agree(name):
    di, x, _, _ = case(name)
    a = DecodeStep(di.wl, x, di.scale, di.sm_scale, fused=True)
    b = DecodeStep(di.wl, x, di.scale, di.sm_scale, fused=False)
    a.select()
    b.select()
    assert np.array_equal(a.sel.cpu().numpy(), b.sel.cpu().numpy())
    assert np.array_equal(a.token_ids.cpu().numpy(), b.token_ids.cpu().numpy())


@pytest.mark.parametrize("name", ALL + SCALE)
def test_selection_chain_general_differs_only_at_the_cutoff(name):
    di, x, ids, nv = case(name)
    step = DecodeStep(di.wl, x, di.scale, di.sm_scale)
    step.select()
    rows = _rows(di, 6)
    rs, rc, sel, _ = _oracle_select(di, ids, nv, rows)
    checks.check_selection(step.sel.cpu().numpy()[rows], sel, rs, rc, _bound(di, rows))


@pytest.mark.parametrize("name", ["tiny", "ragged_bf16", "ragged_prefill", "ragged_fp8",
                                  "fp8_mixed_b32"])
def test_full_path_from_token_cache_exact_twin(name):
    """kpool_compress (fp8 pooling for fp8 workloads) -> compact -> scores -> top-k -> expand
    -> MLA over the paged latent, each side on its own outputs, from the same token-level
    cache: selections and token ids bit-exact with the oracle's chain, and the MLA output
    against the oracle on the same ids. At full size the oracle runs the rows sampled (and
    pools only their sequences)."""
    di = synth.make_decode_inputs(name, exact=True)
    ki = synth.make_kpool_inputs(name, exact=True)
    wl = di.wl
    cfg = config_for(wl)
    x = DeviceDecodeInputs.upload(di)
    k = _dev(ki.k.view(np.int16)).view(torch.bfloat16)
    g = _dev(ki.gate.view(np.int16)).view(torch.bfloat16)
    if wl.key_fp8:
        pk, psc, pv = dsa.kpool_compress_fp8(cfg, k, g, _dev(ki.ape), _dev(ki.valid), wl.first_key)
    else:
        (pk, pv), psc = dsa.kpool_compress(cfg, k, g, _dev(ki.ape), _dev(ki.valid), wl.first_key), None
    del k, g
    x.keys, x.pool_valid, x.key_scales, x.valid = pk, pv, psc, _dev(ki.valid)
    step = DecodeStep(wl, x, di.scale, di.sm_scale)
    step.run()
    rows = _rows(di, 6)
    seqs = np.unique(di.row_seq[rows])
    remap = np.searchsorted(seqs, di.row_seq[rows]).astype(np.int32)
    kk, gg, vv = ki.k[seqs], ki.gate[seqs], np.ascontiguousarray(ki.valid[seqs])
    if wl.key_fp8:
        rk, rks, rv = oracle.kpool_compress_fp8(kk, gg, ki.ape, vv, wl.kpool, wl.first_key)
        assert np.array_equal(psc.cpu().numpy()[seqs], rks)
        assert np.all(rks[rv == 1] == 2.0 ** -8)          # the twin's power-of-two scale
    else:
        (rk, rv), rks = oracle.kpool_compress(kk, gg, ki.ape, vv, wl.kpool, wl.first_key), None
    assert np.array_equal(pv.cpu().numpy()[seqs], rv)
    ids, nv = oracle.compact_pools(rv)
    rs, rc = oracle.index_scores(di.q[rows], di.w[rows], remap, di.row_pos[rows], rk, ids, nv,
                                 kpool=wl.kpool, first_key=wl.first_key, scale=di.scale,
                                 key_scales=rks)
    assert np.array_equal(step.scores.cpu().numpy()[rows].view(np.uint32), rs.view(np.uint32))
    sel = oracle.topk_pools(rs, rc, wl.kw)
    tok = oracle.expand_selection(sel, remap, di.row_pos[rows], vv, kpool=wl.kpool,
                                  index_topk=wl.topk, always_select_tail=wl.tail,
                                  first_key=wl.first_key)
    assert np.array_equal(step.sel.cpu().numpy()[rows], sel)
    gtok = step.token_ids.cpu().numpy()[rows]
    assert np.array_equal(gtok, tok)
    ro, rl = oracle.sparse_mla(di.q_abs[rows], gtok, di.row_seq[rows], di.kv, sm_scale=di.sm_scale,
                               S=wl.S, kv_scales=di.kv_scales, block_table=di.block_table)
    _check_mla(step.out.cpu().numpy()[rows], step.lse.cpu().numpy()[rows], ro, rl, wl.kv_fp8)


@pytest.mark.parametrize("name", ["ragged_fp8", "fp8_mixed_b32"])
def test_decode_step_graph_replay_matches_eager(name):
    di, x, _, _ = case(name)
    step = DecodeStep(di.wl, x, di.scale, di.sm_scale)
    step.run()
    torch.cuda.synchronize()
    ref = (step.sel.clone(), step.token_ids.clone(), step.out.clone(), step.lse.clone())
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step.run()
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(graph):
        step.run()
    for _ in range(3):
        step.out.zero_()
        step.sel.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.sel, ref[0]) and torch.equal(step.token_ids, ref[1])
        assert torch.equal(step.out, ref[2]) and torch.equal(step.lse, ref[3])

"""Comparison rules shared by the GPU parity tests and the CPU tests that show their power.

Tolerances follow the stated correctness rules for the path (index scores within 1e-3
relative, decode outputs within 2e-2 absolute / 1e-2 relative for a bf16 latent and 5e-2 for
fp8, selections differing only at the cutoff), with two additions that keep the checks able to
fail at full size:

* scores: the absolute floor is the a-priori error bound of the f32 arithmetic that computes
  the score (``score_error_bound``), not a fraction of the row's largest score;
* sparse MLA: beside the element-wise rule, each (row, head) must satisfy
  max_c |d| <= 1e-2 * max_c |ref| and ||d||_2 <= 1e-2 * ||ref||_2. Over thousands of nearly
  uniformly weighted latent rows the outputs are a few hundredths, so the element-wise
  absolute floor alone would accept half or twice the right output.
"""
from __future__ import annotations

import numpy as np

import oracle

U32 = 2.0 ** -24          # unit roundoff of binary32

_E4M3 = None


def e4m3_lut() -> np.ndarray:
    global _E4M3
    if _E4M3 is None:
        _E4M3 = np.array([oracle.e4m3_value(c) for c in range(256)], np.float64)
    return _E4M3


def key_values(keys, key_scales=None) -> np.ndarray:
    """Pooled keys as float64 (bf16 bit patterns or e4m3 codes times their row scale)."""
    if keys.dtype == np.uint8:
        v = e4m3_lut()[keys]
        return v * key_scales[..., None].astype(np.float64)
    return (keys.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def score_error_bound(q, w, row_seq, keys, key_scales, scale, rows=None) -> np.ndarray:
    """[R, P] a-priori bound on |f32 score - exact score|.

    The score is sum_h w_h * relu(scale * s_p * dot_h) with dot_h a D-term dot product. In
    binary32, a recursive sum of n terms errs by at most (n - 1) u sum |terms| (u = 2^-24), the
    products of bf16 (or e4m3) operands are exact, each scaling adds one rounding, relu does
    not enlarge an error, and the head sum adds Hi - 1 more. So
    |err| <= (D + Hi + 4) u * sum_h |w_h| |scale s_p| sum_d |q_hd k_pd|; the factor 2 below
    covers second-order terms and accumulation orders with wider intermediates."""
    q = (np.asarray(q).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    R, Hi, D = q.shape
    kv = key_values(keys, key_scales)
    out = np.zeros((R, kv.shape[1]))
    gamma = 2.0 * (D + Hi + 4) * U32
    for r in range(R):
        b = int(row_seq[r])
        if b < 0 or b >= kv.shape[0]:
            continue
        a = np.abs(q[r]) @ np.abs(kv[b]).T                   # [Hi, P]
        out[r] = gamma * abs(scale) * (np.abs(w[r]).astype(np.float64) @ a)
    return out


def check_scores(gs, rs, rc, bound):
    """|gpu - ref| <= 1e-3 |ref| + bound on every candidate slot."""
    for r in range(rs.shape[0]):
        on = rc[r] == 1
        if not on.any():
            continue
        ref = rs[r, on].astype(np.float64)
        got = gs[r, on].astype(np.float64)
        tol = 1e-3 * np.abs(ref) + bound[r, on]
        bad = np.abs(got - ref) > tol
        assert not bad.any(), (r, np.nonzero(on)[0][bad][:5], got[bad][:5], ref[bad][:5])


def check_selection(gsel, sel, rs, rc, bound):
    """Same count per row, GPU picks are candidates listed ascending, and every pool in the
    symmetric difference scores within 1e-3 |cutoff| (plus the two scores' f32 bounds) of
    the oracle's cutoff, the Kw-th best score."""
    for i in range(sel.shape[0]):
        a = set(int(p) for p in sel[i] if p >= 0)
        b = set(int(p) for p in gsel[i] if p >= 0)
        assert len(a) == len(b), (i, len(a), len(b))
        assert all(rc[i, p] for p in b)
        assert list(gsel[i][: len(b)]) == sorted(b)
        diff = a ^ b
        if diff:
            pc = min(a, key=lambda p: (rs[i, p], -p))
            cutoff = float(rs[i, pc])
            for p in diff:
                tol = 1e-3 * abs(cutoff) + bound[i, p] + bound[i, pc]
                assert abs(float(rs[i, p]) - cutoff) <= tol, (i, p, rs[i, p], cutoff)


def mla_errors(go, ro, rl):
    """Per (row, head) with tokens: (max|d| / max|ref|, ||d|| / ||ref||)."""
    d = go.astype(np.float64) - ro
    live = ~np.isneginf(rl)
    mref = np.abs(ro).max(-1)
    lref = np.linalg.norm(ro, axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        rmax = np.where(live, np.abs(d).max(-1) / mref, 0.0)
        rl2 = np.where(live, np.linalg.norm(d, axis=-1) / lref, 0.0)
    return rmax, rl2


def check_mla(go, gl, ro, rl, fp8, rel: float = 1e-2):
    """The stated element-wise rule, the per-(row, head) scale-aware rule, exact zeros for
    rows without tokens, and lse within 1e-4."""
    go = np.asarray(go)
    atol = 5e-2 if fp8 else 2e-2
    err = np.abs(go.astype(np.float64) - ro) - (atol + 1e-2 * np.abs(ro))
    assert err.max() <= 0, ("elementwise", np.unravel_index(err.argmax(), err.shape), err.max())
    assert np.array_equal(np.isneginf(gl), np.isneginf(rl))
    live = ~np.isneginf(rl)
    assert np.all(go[~live] == 0), "a head without tokens must output 0"
    rmax, rl2 = mla_errors(go, ro, rl)
    assert rmax.max() <= rel, ("max|d|/max|ref|", np.unravel_index(rmax.argmax(), rmax.shape),
                               rmax.max())
    assert rl2.max() <= rel, ("L2", np.unravel_index(rl2.argmax(), rl2.shape), rl2.max())
    assert np.allclose(gl[live], rl[live], rtol=1e-4, atol=1e-4)
    return float(rmax.max()), float(rl2.max())

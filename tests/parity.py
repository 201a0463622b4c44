"""Comparison rules between the device path and the oracle (shared by GPU tests).

* fp8 pooled codes: equal, or the two adjacent codes around a rounding midpoint
  where the oracle's pre-rounding value lies within the float32 band of that
  midpoint (the device decides the code in float32, the oracle in float64);
  sigma to 1e-6 relative.
* scores: |S_dev - S_oracle| <= 1e-5 * sum_h |g_h| sum_d |q_hd K_jd| (float32
  accumulation of exact bf16 x fp8 products; 1e-5 is ~20x the float32 bound).
* selection: the rule from the method's acceptance criterion -- ids equal except
  for blocks whose oracle score is within 1e-4 relative of the last kept score.
* attention: max-abs 2e-2 (bf16 outputs) or 1e-5 (f32 outputs).
"""
from __future__ import annotations

import numpy as np

from oracle import oracle as O

ATTN_TOL = {"bf16": 2e-2, "f32": 1e-5}
LSE_TOL = {"bf16": 2e-3, "f32": 1e-5}
SEL_REL = 1e-4


def check_pooled_fp8(g_codes, g_sigma, o_codes, o_sigma, o_v, o_mag, rows):
    gc, oc = g_codes[rows], o_codes[rows]
    np.testing.assert_allclose(g_sigma[rows], o_sigma[rows], rtol=1e-6, atol=0)
    diff = gc != oc
    n = int(diff.sum())
    if n == 0:
        return 0
    r, d = np.nonzero(diff)
    gv = O.fp8_decode(gc[r, d])
    ov = O.fp8_decode(oc[r, d])
    v = o_v[rows][r, d]
    mag = o_mag[rows][r, d]
    mid = (gv + ov) / 2
    band = 1e-5 * (mag + np.abs(v))
    # adjacent: no representable value strictly between the two
    lo, hi = np.minimum(gv, ov), np.maximum(gv, ov)
    allv = np.unique(O.fp8_decode(np.arange(256, dtype=np.uint8)))
    allv = allv[~np.isnan(allv)]
    between = np.array([np.any((allv > a) & (allv < b)) for a, b in zip(lo, hi)])
    ok = (np.abs(v - mid) <= band) & ~between
    assert ok.all(), (
        f"{int((~ok).sum())} pooled codes differ beyond a rounding tie; first at row {rows[r[~ok][0]]} "
        f"dim {d[~ok][0]}: device {gc[r[~ok][0], d[~ok][0]]:#x} oracle {oc[r[~ok][0], d[~ok][0]]:#x} v={v[~ok][0]!r}")
    return n


def check_pooled_f32(g, o, mag, rows):
    err = np.abs(g[rows].astype(np.float64) - o[rows])
    tol = 2e-6 * mag[rows] + 1e-30
    assert np.all(err <= tol), f"pooled f32 max err {err.max()} (tol {tol[np.argmax(err - tol)]})"


def score_bound(q_idx, gates, keys):
    """sum_h |g_h| sum_d |q_hd K_jd| for every key."""
    return np.abs(np.asarray(keys, np.float64)) @ np.abs(np.asarray(q_idx, np.float64)).T @ np.abs(gates)


def check_scores(g_scores, o_scores, q_idx, gates, keys):
    bound = score_bound(q_idx, gates, keys)
    err = np.abs(np.asarray(g_scores, np.float64) - o_scores)
    ok = err <= 1e-5 * bound + 1e-30
    assert ok.all(), f"{int((~ok).sum())} scores off; worst rel {(err / (bound + 1e-30)).max():.3e}"


def check_selection(g_ids, o_ids, o_scores, b_q, k):
    """Acceptance rule for one row (see module docstring)."""
    g_ids = np.asarray(g_ids)
    o_ids = np.asarray(o_ids)
    kp = min(k, b_q + 1)
    # format: kp valid ids ascending, the own block last among them, then -1
    assert np.all(g_ids[kp:] == -1), "padding"
    gv = g_ids[:kp]
    assert np.all(gv >= 0) and np.all(np.diff(gv) > 0), "ids must be ascending and valid"
    assert gv[-1] == b_q, "own block missing"
    if np.array_equal(g_ids, o_ids):
        return 0
    ov = o_ids[:kp]
    S = np.asarray(o_scores, np.float64)
    # the k-th score: the smallest score among the kept eligible blocks
    s_star = S[ov[:-1]].min() if kp >= 2 else 0.0
    near = set(np.nonzero(np.abs(S - s_star) <= SEL_REL * abs(s_star))[0].tolist())
    gs, os_ = set(gv.tolist()), set(ov.tolist())
    assert (gs - near) == (os_ - near), (
        f"selection differs outside the tie band: extra {sorted((gs - os_) - near)[:8]}, "
        f"missing {sorted((os_ - gs) - near)[:8]}")
    return len(gs ^ os_)


def check_attention(g_out, o_out, kind):
    err = np.abs(np.asarray(g_out, np.float64) - o_out)
    assert err.max() <= ATTN_TOL[kind], f"attention max-abs {err.max():.3e} > {ATTN_TOL[kind]}"
    return float(err.max())


def check_lse(g_lse, o_lse, kind):
    err = np.abs(np.asarray(g_lse, np.float64) - o_lse)
    assert err.max() <= LSE_TOL[kind], f"lse max-abs {err.max():.3e} > {LSE_TOL[kind]}"

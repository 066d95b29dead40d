"""Comparison rules between the GPU path and the oracle.

Scores (fp32 accumulation on the GPU, fp64 in the oracle): for query row q
let rho = RMS of the oracle's scores over the valid rows; every valid score
must satisfy |g - o| <= 1e-2 * max(|o|, f rho), f = 1 in general and 1e-3
for layers of at least 32 heads whose head weights are all non-negative.  The floor keeps
exact-zero scores (a row whose every head is cut by the ReLU) well defined;
with mixed-sign weights, heads can cancel a score to near zero, which only
an absolute bound can judge.

Top-k sets: the GPU set has the right size, no duplicates and only valid
positions; every position the oracle picked that the GPU left out, and every
position the GPU picked that the oracle left out, must lie within one
tolerance band of the oracle's cut-off score, i.e.
max(o over missed) - min(o over extra) < 1e-2 * max(|t|, rho), t = the
oracle's smallest selected score.  Exactly equal scores may be swapped
freely; that is why several GPU answers can be correct.
"""
from __future__ import annotations

import numpy as np

REL_TOL = 1e-2


def rms(x: np.ndarray) -> float:
    x = np.asarray(x, dtype=np.float64)
    return float(np.sqrt(np.mean(x * x))) if x.size else 0.0


# Stricter floor for layers of many heads whose head weights are all
# non-negative: there every head adds a non-negative term, a score is small
# only when every head is small, and its error stays relative to it; the
# RMS floor then only covers near-zero scores (every head cut or nearly so
# by the ReLU).
STRICT_FLOOR = 1e-3


def check_scores(g: np.ndarray, o: np.ndarray, what: str = "scores", floor_frac: float = 1.0) -> float:
    """Assert |g - o| <= 1e-2 max(|o|, floor_frac rho) for every row; returns
    the worst purely relative error |g - o| / |o| over the rows with
    |o| >= 1e-3 rho (reported by the tests).  floor_frac = 1 is the general
    rule (mixed-sign head weights can cancel a score to near zero, where only
    an absolute bound is meaningful); STRICT_FLOOR is used for non-negative
    head weights."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    assert g.shape == o.shape, (what, g.shape, o.shape)
    if o.size == 0:
        return 0.0
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU scores"
    rho = max(rms(o), 1e-30)
    den = np.maximum(np.abs(o), floor_frac * rho)
    err = np.abs(g - o) / den
    worst = float(err.max())
    if worst > REL_TOL:
        i = int(err.argmax())
        raise AssertionError(f"{what}: row {i} gpu={g[i]!r} oracle={o[i]!r} rel={worst:.3e} > {REL_TOL} "
                             f"(floor {floor_frac:g} x RMS)")
    big = np.abs(o) >= STRICT_FLOOR * rho
    return float((np.abs(g - o)[big] / np.abs(o[big])).max()) if big.any() else 0.0


def check_topk(gsel: np.ndarray, gcount: int, oracle_sel: np.ndarray, o_scores_by_pos: dict | np.ndarray,
               valid: np.ndarray | None, K: int, rho: float, what: str = "top-k") -> int:
    """Assert the top-k rule.

    gsel: the GPU's row of positions (length k, -1 padded); gcount: its count.
    oracle_sel: the oracle's selected positions.  o_scores_by_pos: oracle
    score of any valid position (array indexed by position, or dict).
    valid: allowed positions (None: 0..len(scores)-1).  Returns the number of
    tolerated swaps.
    """
    assert gcount == K, f"{what}: count {gcount} != {K}"
    gs = np.asarray(gsel[:K], dtype=np.int64)
    assert np.all(np.asarray(gsel[K:]) == -1), f"{what}: padding is not -1"
    assert len(np.unique(gs)) == K, f"{what}: duplicate positions"
    if isinstance(o_scores_by_pos, dict):
        sc = o_scores_by_pos
        score = lambda p: sc[int(p)]
        if valid is None:
            valid = np.fromiter(sc.keys(), dtype=np.int64)
    else:
        arr = np.asarray(o_scores_by_pos, dtype=np.float64)
        score = lambda p: arr[int(p)]
        if valid is None:
            valid = np.arange(arr.size)
    vset = set(np.asarray(valid, dtype=np.int64).tolist())
    bad = [int(p) for p in gs if int(p) not in vset]
    assert not bad, f"{what}: positions outside the valid set: {bad[:5]}"
    os_ = set(np.asarray(oracle_sel, dtype=np.int64).tolist())
    assert len(os_) == K, f"{what}: oracle picked {len(os_)} != {K}"
    gset = set(gs.tolist())
    missed = os_ - gset
    extra = gset - os_
    assert len(missed) == len(extra)
    if not missed:
        return 0
    t = min(score(p) for p in os_)
    band = REL_TOL * max(abs(t), rho)
    hi = max(score(p) for p in missed)
    lo = min(score(p) for p in extra)
    assert hi - lo < band or hi - lo <= 0.0, \
        f"{what}: {len(missed)} swaps, missed score {hi!r} vs extra {lo!r} beyond band {band!r}"
    return len(missed)


def overlap(a: np.ndarray, b: np.ndarray) -> float:
    sa, sb = set(np.asarray(a).tolist()), set(np.asarray(b).tolist())
    return len(sa & sb) / max(1, len(sb))

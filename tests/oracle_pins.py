"""Pins of the CPU oracle to facts outside itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
something the LatentIndex paper (paperlayer.ai summary of arXiv:2610.04635)
or plain mathematics fixes: hand-derived worked examples (tests/golden/),
the absorption identity (§3.1: exact for the effective keys in exact
arithmetic), special cases that reduce to a textbook dot product or a
library sort, brute-force selection on tiny inputs, the HS reductions named
for the method (M >= n gives full LatentIndex, M = k gives index reuse) and
the closed forms of §3.4/§B.1/§B.3.

``test_oracle.py`` runs every pin on the real oracle and on deliberately
broken copies of it, so each pin is known to catch the mistakes it targets.
"""
from __future__ import annotations

import itertools
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------
# Worked examples
# ----------------------------------------------------------------------------
def pin_worked_absorb():
    g = _golden("worked_score_topk.json")
    qt = oracle.absorb(np.array(g["q"], float), np.array(g["W_dec"], float))
    assert np.array_equal(qt, np.array(g["absorbed"], float)), qt


def pin_worked_scores():
    g = _golden("worked_score_topk.json")
    qt = np.array(g["absorbed"], float)
    s = oracle.score(qt, np.array(g["w"], float), np.array(g["latent"], float))
    assert np.array_equal(s, np.array(g["scores"], float)), s
    # the same rows listed explicitly, out of order
    rows = np.array([4, 0, 2], dtype=np.int32)
    s2 = oracle.score(qt, np.array(g["w"], float), np.array(g["latent"], float), rows=rows)
    assert np.array_equal(s2, np.array(g["scores"], float)[rows]), s2


def pin_worked_explicit_keys():
    g = _golden("worked_score_topk.json")
    s = oracle.score_explicit(np.array(g["q"], float), np.array(g["W_dec"], float), np.array(g["w"], float),
                              np.array(g["latent"], float))
    assert np.array_equal(s, np.array(g["scores"], float)), s


def pin_worked_topk():
    g = _golden("worked_score_topk.json")
    s = np.array(g["scores"], float)
    order = g["topk_order"]
    for K in range(0, len(order) + 2):
        got = oracle.topk(s, K)
        assert list(got) == order[:K], (K, got)


def pin_worked_causal():
    g = _golden("worked_score_topk.json")
    q = np.array(g["q"], float)
    W = np.array(g["W_dec"], float)
    w = np.array(g["w"], float)
    C = np.array(g["latent"], float)
    for case in g["causal"]:
        n = oracle.valid_rows(case["pos"], C.shape[0])
        assert n == case["n_valid"], (case, n)
        res = oracle.full_layer(q[None], W, w[None], [C], np.array([0]), np.array([case["pos"]]),
                                np.array([C.shape[0]]), case["k"])
        assert sorted(res[0].sel.tolist()) == sorted(case["selected"]), (case, res[0].sel)


def pin_worked_hs():
    g = _golden("worked_hs.json")
    C = np.array(g["latent"], float)
    I = np.eye(2)
    qa, wa = np.array(g["anchor"]["q"], float), np.array(g["anchor"]["w"], float)
    qf, wf = np.array(g["follower"]["q"], float), np.array(g["follower"]["w"], float)
    assert np.array_equal(oracle.score(qa, wa, C), np.array(g["anchor_scores"], float))
    assert np.array_equal(oracle.score(qf, wf, C), np.array(g["follower_scores"], float))
    n = C.shape[0]
    for case in g["cases"]:
        res = oracle.hs_group([qa[None], qf[None]], [I, I], [wa[None], wf[None]], [C], np.array([0]),
                              np.array([n - 1]), np.array([n]), case["k"], case["M"])
        assert res[0][0].cand.tolist() == case["cand"], (case, res[0][0].cand)
        assert res[0][0].sel.tolist() == case["anchor_sel"], (case, res[0][0].sel)
        assert res[1][0].sel.tolist() == case["follower_sel"], (case, res[1][0].sel)
    full = oracle.full_layer(qf[None], I, wf[None], [C], np.array([0]), np.array([n - 1]), np.array([n]), 2)
    assert full[0].sel.tolist() == g["full_follower_sel_k2"]


# ----------------------------------------------------------------------------
# Identities and special cases
# ----------------------------------------------------------------------------
def _rand_case(rng, H, d, r, n):
    q = rng.standard_normal((H, d))
    W = rng.standard_normal((d, r)) / np.sqrt(r)
    w = rng.random(H) + 0.1
    C = rng.standard_normal((n, r))
    return q, W, w, C


def pin_absorption_identity():
    """Scores from absorbed queries equal scores from rebuilt keys (§3.1)."""
    rng = np.random.default_rng(11)
    for (H, d, r, n) in [(4, 32, 64, 200), (3, 5, 7, 50), (8, 16, 12, 64)]:
        q, W, w, C = _rand_case(rng, H, d, r, n)
        a = oracle.score(oracle.absorb(q, W), w, C)
        b = oracle.score_explicit(q, W, w, C)
        scale = np.max(np.abs(a)) + 1.0
        assert np.max(np.abs(a - b)) <= 1e-12 * scale, (H, d, r, np.max(np.abs(a - b)))
        assert np.count_nonzero(a) > 0


def pin_absorb_matches_matmul():
    """Absorption is a matrix product: compare with numpy's (library routine)."""
    rng = np.random.default_rng(12)
    q = rng.standard_normal((3, 4, 5))
    W = rng.standard_normal((5, 9))
    got = oracle.absorb(q, W)
    ref = np.matmul(q, W)
    assert got.shape == (3, 4, 9)
    assert np.max(np.abs(got - ref)) <= 1e-12 * (np.max(np.abs(ref)) + 1), np.max(np.abs(got - ref))


def pin_one_hot_head_is_relu_dot():
    """w = e_h reduces the score to max(0, qt_h . c) (a textbook dot product)."""
    rng = np.random.default_rng(13)
    H, r, n = 5, 11, 40
    qt = rng.standard_normal((H, r))
    C = rng.standard_normal((n, r))
    for h in range(H):
        w = np.zeros(H)
        w[h] = 1.0
        got = oracle.score(qt, w, C)
        ref = np.maximum(0.0, C @ qt[h])
        assert np.max(np.abs(got - ref)) <= 1e-12 * (np.max(np.abs(ref)) + 1), h


def pin_identity_decoder_is_per_layer_indexer():
    """With W_dec = I (r = d) a group of one is the native per-layer indexer."""
    rng = np.random.default_rng(14)
    H, d, n = 6, 16, 80
    q = rng.standard_normal((H, d))
    w = rng.standard_normal(H)
    K = rng.standard_normal((n, d))
    qt = oracle.absorb(q, np.eye(d))
    assert np.array_equal(qt, q)
    a = oracle.score(qt, w, K)
    b = oracle.score_explicit(q, None, w, K)
    assert np.max(np.abs(a - b)) <= 1e-12 * (np.max(np.abs(a)) + 1)


def pin_homogeneity_and_permutation():
    """ReLU is positively homogeneous; heads are an unordered sum."""
    rng = np.random.default_rng(15)
    H, r, n = 7, 9, 60
    qt = rng.standard_normal((H, r))
    w = rng.standard_normal(H)
    C = rng.standard_normal((n, r))
    s = oracle.score(qt, w, C)
    assert np.allclose(oracle.score(qt, w, 2.0 * C), 2.0 * s, rtol=1e-13, atol=1e-13)
    assert np.allclose(oracle.score(qt, 3.0 * w, C), 3.0 * s, rtol=1e-13, atol=1e-13)
    perm = rng.permutation(H)
    assert np.allclose(oracle.score(qt[perm], w[perm], C), s, rtol=1e-13, atol=1e-13)
    # a head whose dot is negative everywhere contributes nothing
    qn = np.vstack([qt, -np.ones((1, r))])
    Cp = np.abs(C)
    wn = np.append(w, 5.0)
    assert np.allclose(oracle.score(qn, wn, Cp), oracle.score(qt, w, Cp), rtol=1e-13, atol=1e-13)
    # negative head weights subtract
    w1 = np.zeros(H)
    w1[0] = -2.0
    assert np.allclose(oracle.score(qt, w1, C), -2.0 * np.maximum(0, C @ qt[0]), rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------------------------
# Selection
# ----------------------------------------------------------------------------
def _dominates(si, pi, sj, pj):
    return si > sj or (si == sj and pi < pj)


def pin_topk_brute_force():
    """Top-K is the unique K-subset every member of which beats every outsider."""
    rng = np.random.default_rng(16)
    for trial in range(60):
        n = int(rng.integers(1, 9))
        s = rng.integers(0, 4, size=n).astype(float) * 0.5   # many exact ties
        if trial % 3 == 0:
            s = rng.standard_normal(n)
        for K in range(0, n + 2):
            Ke = min(K, n)
            winners = []
            for sub in itertools.combinations(range(n), Ke):
                inside = set(sub)
                ok = all(_dominates(s[i], i, s[j], j) for i in inside for j in range(n) if j not in inside)
                if ok:
                    winners.append(set(sub))
            assert len(winners) == 1
            got = oracle.topk(s, K)
            assert len(got) == Ke and set(got.tolist()) == winners[0], (s, K, got)
            # the order is score descending, position ascending
            for a, b in zip(got[:-1], got[1:]):
                assert _dominates(s[a], a, s[b], b)


def pin_topk_matches_lexsort():
    """Same result as numpy's lexsort on (-score, position)."""
    rng = np.random.default_rng(17)
    for n in (1, 5, 100, 1000):
        s = np.round(rng.standard_normal(n), 1)
        pos = rng.permutation(10 * n)[:n].astype(np.int32)
        order = np.lexsort((pos, -s))
        for K in (0, 1, n // 3, n, n + 5):
            got = oracle.topk(s, K, pos=pos)
            assert np.array_equal(got, pos[order[:min(K, n)]]), (n, K)


def pin_topk_invariants():
    rng = np.random.default_rng(18)
    s = rng.standard_normal(5000)
    s[::7] = 0.0
    for K in (1, 64, 2048, 4999, 5000):
        got = oracle.topk(s, K)
        assert len(got) == K and len(set(got.tolist())) == K
        mask = np.zeros(5000, bool)
        mask[got] = True
        if K < 5000:
            assert s[mask].min() >= s[~mask].max()


# ----------------------------------------------------------------------------
# Hierarchical selection reductions
# ----------------------------------------------------------------------------
def _group(rng, G=4, H=3, d=6, r=8, lens=(50, 37)):
    B = len(lens)
    lat = [rng.standard_normal((n, r)) for n in lens]
    q = [rng.standard_normal((B, H, d)) for _ in range(G)]
    W = [rng.standard_normal((d, r)) / np.sqrt(r) for _ in range(G)]
    w = [rng.random((B, H)) + 0.05 for _ in range(G)]
    qseq = np.arange(B)
    qpos = np.array(lens) - 1
    return q, W, w, lat, qseq, qpos, np.array(lens)


def pin_hs_full_budget_is_full_latentindex():
    """M >= n: HS selects exactly what full LatentIndex selects, in every layer."""
    rng = np.random.default_rng(19)
    q, W, w, lat, qseq, qpos, lens = _group(rng)
    k = 10
    hs = oracle.hs_group(q, W, w, lat, qseq, qpos, lens, k, M=1000)
    for l in range(len(q)):
        full = oracle.full_layer(q[l], W[l], w[l], lat, qseq, qpos, lens, k)
        for i in range(len(qseq)):
            assert np.array_equal(hs[l][i].sel, full[i].sel), (l, i)


def pin_hs_budget_k_is_index_reuse():
    """M = k: every follower returns the anchor's own selection (IndexCache reuse)."""
    rng = np.random.default_rng(20)
    q, W, w, lat, qseq, qpos, lens = _group(rng)
    k = 7
    hs = oracle.hs_group(q, W, w, lat, qseq, qpos, lens, k, M=k)
    for i in range(len(qseq)):
        anchor = set(hs[0][i].sel.tolist())
        for l in range(1, len(q)):
            assert set(hs[l][i].sel.tolist()) == anchor, (l, i)


def pin_hs_subsets_and_caps():
    rng = np.random.default_rng(21)
    q, W, w, lat, qseq, qpos, lens = _group(rng, lens=(40, 9))
    k, M = 6, 12
    hs = oracle.hs_group(q, W, w, lat, qseq, qpos, lens, k, M)
    for i in range(len(qseq)):
        n = int(lens[i])
        cand = hs[0][i].cand
        assert len(cand) == min(M, n) and len(set(cand.tolist())) == len(cand)
        assert set(hs[0][i].sel.tolist()) <= set(cand.tolist())
        for l in range(1, len(q)):
            sel = hs[l][i].sel
            assert len(sel) == min(k, len(cand))
            assert set(sel.tolist()) <= set(cand.tolist())
            # the follower's pick is its own top-k within the candidates
            s_all = oracle.score(oracle.absorb(q[l][i], W[l]), w[l][i], lat[i], n)
            ref = oracle.topk(s_all[cand], k, pos=cand)
            assert np.array_equal(sel, ref)


# ----------------------------------------------------------------------------
# Closed forms
# ----------------------------------------------------------------------------
def pin_scored_positions():
    """§3.4: a group of m layers scores L + (m-1) min(B, L); §B.3: 16L + 45*8192 vs 61L."""
    g = _golden("closed_forms.json")["positions"]
    rng = np.random.default_rng(22)
    q, W, w, lat, qseq, qpos, lens = _group(rng, lens=(30, 5))
    M = 12
    hs = oracle.hs_group(q, W, w, lat, qseq, qpos, lens, 4, M)
    G = len(q)
    for i in range(len(qseq)):
        n = int(lens[i])
        got = oracle.rows_scored_hs(n, len(hs[1][i].cand_scores), G)
        assert got == n + (G - 1) * min(M, n), (n, got)
        assert oracle.rows_scored_full(n, G) == G * n
    for L in (8193, 16384, 65536, 131072):
        hs_pos = oracle.model_positions_hs(L, g["independent"], g["groups"], g["G"], g["M"])
        assert hs_pos == 16 * L + 45 * 8192, L
        dsa = oracle.model_positions_hs(L, g["n_layers"], 0, g["G"], g["M"])
        assert dsa == 61 * L


def pin_storage_accounting():
    """§3.4/§B.1: 8052 -> 3132 bytes per token, a 61.1% cut at G=4."""
    g = _golden("closed_forms.json")["storage"]
    dsa, grouped = oracle.storage_bytes_per_token(g["n_layers"], g["groups"], g["G"], 132, 200)
    assert dsa == g["dsa_bytes"] and grouped == g["grouped_bytes"], (dsa, grouped)
    assert round(100.0 * (1 - grouped / dsa), 1) == g["reduction_pct_1dp"]


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]

"""Pins of the CPU oracle to facts outside itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
something the LatentIndex paper (paperlayer.ai summary of arXiv:2610.04635)
or plain mathematics fixes: hand-derived worked examples (tests/golden/),
the absorption identity (§3.1: scores from the absorbed query equal scores
through the explicitly decoded keys, up to rounding), special cases that reduce to a textbook dot product or a
library sort, brute-force selection on tiny inputs, the HS reductions named
for the method (M >= n gives full LatentIndex, M = k gives index reuse) and
the closed forms of §3.4/§B.1/§B.3.

``test_oracle.py`` runs every pin on the real oracle and on deliberately
broken copies of it, so each pin is known to catch the mistakes it targets.
"""
from __future__ import annotations

import itertools
import math
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


def pin_worked_baseline_layer():
    """The per-layer indexer on its own cached keys (no decoder): with the
    keys rebuilt by hand from the worked latent it gives the latent path's
    scores and selection, causal prefix included."""
    g = _golden("worked_score_topk.json")
    q = np.array(g["q"], float)[None]
    w = np.array(g["w"], float)[None]
    K = np.array(g["keys"], float)
    res = oracle.baseline_layer(q, w, [K], np.array([0]), np.array([4]), np.array([5]), 3)
    assert np.array_equal(res[0].scores, np.array(g["scores"], float)), res[0].scores
    assert list(res[0].sel) == g["topk_order"][:3], res[0].sel
    for case in g["causal"]:
        res = oracle.baseline_layer(q, w, [K], np.array([0]), np.array([case["pos"]]), np.array([5]), case["k"])
        assert len(res[0].scores) == case["n_valid"] and sorted(res[0].sel) == case["selected"], (case, res[0].sel)


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


# ----------------------------------------------------------------------------
# Segmented FP8 (OCP E4M3 codes, Walsh-Hadamard rotation, power-of-two scales)
# ----------------------------------------------------------------------------
def _finite_codes():
    return np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def _e4m3_value(c: int) -> float:
    """Value of a code straight from the format definition (independent of the oracle)."""
    s = -1.0 if c & 0x80 else 1.0
    E, m = (c >> 3) & 15, c & 7
    return s * (m / 8.0 * 2.0 ** -6 if E == 0 else (1.0 + m / 8.0) * 2.0 ** (E - 7))


def pin_e4m3_code_table():
    g = _golden("worked_fp8.json")
    for c, v in g["code_values"]:
        got = float(oracle.e4m3_decode([c])[0])
        assert got == v and np.signbit(got) == np.signbit(v), (c, got, v)
    codes = _finite_codes()
    vals = oracle.e4m3_decode(codes)
    assert all(vals[i] == _e4m3_value(int(c)) for i, c in enumerate(codes))


def pin_e4m3_encode_worked_cases():
    g = _golden("worked_fp8.json")
    for v, c, why in g["encode_cases"]:
        got = int(oracle.e4m3_encode([v])[0])
        assert got == c, (v, got, c, why)


def pin_e4m3_roundtrip():
    codes = _finite_codes()
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


def pin_e4m3_encode_brute_force():
    """Nearest code by exhaustive search, ties to the even mantissa, saturation at 448."""
    codes = _finite_codes()
    table = np.array([_e4m3_value(int(c)) for c in codes])
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(400) * 10.0 ** rng.uniform(-4, 3, 400),
                        (rng.integers(-3000, 3000, 300) / 8.0) * 2.0 ** rng.integers(-12, 6, 300)]).astype(np.float32)
    got = oracle.e4m3_encode(x)
    for v, c in zip(x.astype(np.float64), got):
        if abs(v) >= 448.0:
            want = 0xFE if v < 0 else 0x7E
        else:
            d = np.abs(table - v)
            best = np.flatnonzero(d == d.min())
            cand = [int(codes[i]) for i in best]
            if len(cand) > 1:  # a tie: keep codes of the sign of v, then the even mantissa
                same = [k for k in cand if bool(k & 0x80) == bool(np.signbit(v))] or cand
                cand = [k for k in same if (k & 7) % 2 == 0] or same
            want = cand[0]
        assert _e4m3_value(int(c)) == _e4m3_value(want), (float(v), int(c), want)


def pin_wht_is_the_normalized_hadamard_matrix():
    """Sylvester Hadamard matrix / sqrt(128), to fp32 accuracy; orthonormal and self-inverse."""
    Hm = np.array([[1.0]])
    while Hm.shape[0] < 128:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    Hm /= np.sqrt(128.0)
    rng = np.random.default_rng(8)
    for _ in range(5):
        x = rng.standard_normal(128).astype(np.float32)
        y = oracle.wht128(x)
        ref = Hm @ x.astype(np.float64)
        assert np.max(np.abs(y - ref)) <= 1e-5 * (1 + np.max(np.abs(ref))), np.max(np.abs(y - ref))
        back = oracle.wht128(y)
        assert np.max(np.abs(back - x)) <= 1e-5 * (1 + np.max(np.abs(x)))
        assert abs(np.linalg.norm(y.astype(np.float64)) - np.linalg.norm(x.astype(np.float64))) <= 1e-5 * np.linalg.norm(x)


def pin_pow2_exponent():
    g = _golden("worked_fp8.json")
    for a, e in g["pow2_cases"]:
        assert oracle.pow2_exponent(a) == e, (a, oracle.pow2_exponent(a), e)
    rng = np.random.default_rng(9)
    for a in (10.0 ** rng.uniform(-20, 20, 300)).astype(np.float32):
        e = oracle.pow2_exponent(a)
        assert float(a) * 2.0 ** -e <= 448.0 < float(a) * 2.0 ** -(e - 1), (a, e)


def pin_quantize_worked_examples():
    g = _golden("worked_fp8.json")
    row = np.zeros((1, 128), np.float32)
    row[0, 0] = 1.0
    c, s = oracle.quantize_rows(row)
    ex = g["quantize_e0"]
    assert s[0, 0] == ex["scale"] == 2.0 ** ex["exponent"] and np.all(c == ex["code"]), (s, c[0, :4])
    row[0, 1] = 1.0
    c, s = oracle.quantize_rows(row)
    ex = g["quantize_e0_e1"]
    assert s[0, 0] == 2.0 ** ex["exponent"]
    assert np.all(c[0, 0::2] == ex["code_even"]) and np.all(c[0, 1::2] == ex["code_odd"])
    # two segments are quantized independently
    two = np.zeros((1, 256), np.float32)
    two[0, 0], two[0, 128] = 1.0, 4.0
    c2, s2 = oracle.quantize_rows(two)
    assert s2[0, 0] == 2.0 ** -12 and s2[0, 1] == 2.0 ** -10 and np.all(c2 == 123)


def worked_absorb_fp8_operands(r=128):
    """q [1][1][32] and W [32][r] of the worked FP8 absorption case."""
    g = _golden("worked_fp8.json")["absorb_case"]
    q = np.zeros((1, 1, 32), np.float32)
    q[0, 0, :len(g["q_terms"])] = g["q_terms"]
    W = np.zeros((32, r), np.float32)
    W[:len(g["w_column0"]), 0] = g["w_column0"]
    return q, W


def pin_worked_absorb_fp8():
    """The absorbed query is the exact product rounded once to fp32 before the
    rotation: here that one rounding decides every code of the segment."""
    g = _golden("worked_fp8.json")["absorb_case"]
    for r in (128, 256):
        q, W = worked_absorb_fp8_operands(r)
        codes, scales = oracle.absorb_fp8(q, W)
        assert codes.shape == (1, 1, r) and scales.shape == (1, 1, r // 128)
        assert scales[0, 0, 0] == g["scale"] == 2.0 ** g["exponent"], scales
        assert np.all(codes[0, 0, :128] == g["code"]), codes[0, 0, :8]
        if r == 256:  # an all-zero segment: exponent 0, zero codes
            assert scales[0, 0, 1] == 1.0 and not codes[0, 0, 128:].any()
    # the next float32 below x (any rounding of x other than to nearest)
    row = np.zeros((1, 128), np.float32)
    row[0, 0] = np.float32(8526734 * 2.0 ** -23)
    c, s = oracle.quantize_rows(row)
    assert s[0, 0] == g["scale"] and np.all(c == g["code_if_x_rounded_down"]), c[0, :4]


def pin_quantization_error_bound():
    """Each dequantized element is within half a step of its rotated value."""
    rng = np.random.default_rng(10)
    x = (rng.standard_normal((6, 256)) * rng.uniform(0.01, 100, (6, 1))).astype(np.float32)
    c, s = oracle.quantize_rows(x)
    for i in range(6):
        for gseg in range(2):
            y = oracle.wht128(x[i, gseg * 128:(gseg + 1) * 128]).astype(np.float64)
            d = oracle.e4m3_decode(c[i, gseg * 128:(gseg + 1) * 128]) * float(s[i, gseg])
            step = np.maximum(np.abs(y) * 2.0 ** -3, 2.0 ** -9 * float(s[i, gseg]))
            assert np.all(np.abs(d - y) <= step / 2 * (1 + 1e-12)), np.max(np.abs(d - y) / step)
            assert np.max(np.abs(d)) <= 448.0 * float(s[i, gseg])


def pin_fp8_score_worked_case():
    g = _golden("worked_fp8.json")["score_case"]
    e0 = np.zeros((1, 128), np.float32)
    e0[0, 0] = 1.0
    qc, qs = oracle.quantize_rows(e0)
    cc_pos, cs_pos = oracle.quantize_rows(e0)
    cc_neg, cs_neg = oracle.quantize_rows(-e0)
    cc = np.concatenate([cc_pos, cc_neg])
    cs = np.concatenate([cs_pos, cs_neg])
    s = oracle.score_fp8(qc, qs, np.array(g["w"]), cc, cs)
    assert s[0] == g["score_pos"] and s[1] == g["score_neg"], s


def pin_fp8_score_is_plain_score_of_dequantized_rows():
    """Reduces to the (pinned) plain scorer on the dequantized, scaled rows."""
    rng = np.random.default_rng(11)
    H, r, n = 5, 256, 40
    q = rng.standard_normal((H, r)).astype(np.float32)
    C = rng.standard_normal((n, r)).astype(np.float32)
    w = rng.uniform(-1, 1, H)
    qc, qs = oracle.quantize_rows(q)
    cc, cs = oracle.quantize_rows(C)
    qd = oracle.e4m3_decode(qc) * np.repeat(qs.astype(np.float64), 128, axis=1)
    cd = oracle.e4m3_decode(cc) * np.repeat(cs.astype(np.float64), 128, axis=1)
    want = oracle.score(qd, w, cd)
    got = oracle.score_fp8(qc, qs, w, cc, cs)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.max(np.abs(want))), np.max(np.abs(got - want))
    rows = np.array([7, 3, 39, 0], dtype=np.int32)
    assert np.array_equal(oracle.score_fp8(qc, qs, w, cc, cs, rows=rows), got[rows])


def pin_rotation_keeps_the_score():
    """The orthonormal rotation alone changes no score beyond fp32 rounding."""
    rng = np.random.default_rng(12)
    H, r, n = 4, 256, 30
    q = rng.standard_normal((H, r)).astype(np.float32)
    C = rng.standard_normal((n, r)).astype(np.float32)
    w = rng.uniform(0, 1, H)
    rot = lambda a: np.concatenate([oracle.wht128(a[g * 128:(g + 1) * 128]) for g in range(2)])
    qr = np.stack([rot(x) for x in q])
    cr = np.stack([rot(x) for x in C])
    a, b = oracle.score(q, w, C), oracle.score(qr, w, cr)
    assert np.max(np.abs(a - b)) <= 1e-4 * (1 + np.max(np.abs(a)))


# ----------------------------------------------------------------------------
# RoPE-compatible structured decoder (§A.2-§A.4)
# ----------------------------------------------------------------------------
def pin_worked_absorb_rope():
    g = _golden("worked_rope.json")["absorb"]
    qt, b = oracle.absorb_rope(np.array([g["q"]]), np.array(g["D"]), np.array(g["Wn"]), np.array(g["beta"]), 1, 1)
    assert np.array_equal(qt[0], np.array(g["qt"])), qt
    assert b[0] == g["bias"], b


def pin_worked_rope_rotation():
    g = _golden("worked_rope.json")["rotation"]
    th = g["theta"]
    p = g["pos"]
    c0, s0 = math.cos(p * th[0]), math.sin(p * th[0])
    c1, s1 = math.cos(p * th[1]), math.sin(p * th[1])
    want = np.array([c0, s0, -s1, c1, 2 * c0, 2 * s0, 0.0, 0.0, 5.0])
    got = oracle.rope_rotate(np.array([g["row"]]), np.array([p]), g["F"], g["S"], g["base"])[0]
    assert np.allclose(got, want, rtol=0, atol=1e-15), (got, want)


def pin_rope_zero_position_composition_and_norm():
    rng = np.random.default_rng(21)
    F, S, rn = 8, 2, 5
    X = rng.standard_normal((6, 2 * S * F + rn))
    assert np.array_equal(oracle.rope_rotate(X, np.zeros(6), F, S), X)
    p1 = rng.integers(0, 60000, 6)
    p2 = rng.integers(0, 60000, 6)
    twice = oracle.rope_rotate(oracle.rope_rotate(X, p1, F, S), p2, F, S)
    once = oracle.rope_rotate(X, p1 + p2, F, S)
    assert np.allclose(twice, once, rtol=0, atol=1e-9)
    Y = oracle.rope_rotate(X, p1, F, S)
    pr = lambda Z: np.hypot(Z[:, 0:2 * S * F:2], Z[:, 1:2 * S * F:2])
    assert np.allclose(pr(Y), pr(X), rtol=1e-14, atol=0)
    assert np.array_equal(Y[:, 2 * S * F:], X[:, 2 * S * F:])


def _rope_case(rng, H=3, F=4, S=2, dn=6, rn=8, n=60):
    q = rng.standard_normal((H, 2 * F + dn))
    D = rng.standard_normal((F, S, 2))
    Wn = rng.standard_normal((dn, rn))
    beta = rng.standard_normal(dn)
    w = rng.random(H) + 0.1
    C = rng.standard_normal((n, 2 * S * F + rn))
    pos = rng.integers(0, 131072, n)
    return q, D, Wn, beta, w, C, pos


def pin_rope_absorption_identity():
    rng = np.random.default_rng(22)
    for (F, S, dn, rn) in ((4, 2, 6, 8), (3, 1, 5, 4), (6, 3, 2, 7)):
        q, D, Wn, beta, w, C, pos = _rope_case(rng, F=F, S=S, dn=dn, rn=rn)
        qt, b = oracle.absorb_rope(q, D, Wn, beta, F, S)
        latent = oracle.score(qt, w, oracle.rope_rotate(C, pos, F, S), bias=b)
        explicit = oracle.score_explicit_rope(q, D, Wn, beta, w, C, pos, F, S)
        assert np.allclose(latent, explicit, rtol=1e-11, atol=1e-11), np.max(np.abs(latent - explicit))
        assert np.mean(latent > 0) > 0.5


def pin_rope_without_rotary_part_is_plain_absorption():
    rng = np.random.default_rng(23)
    q = rng.standard_normal((2, 3, 5))
    Wn = rng.standard_normal((5, 7))
    qt, b = oracle.absorb_rope(q, np.zeros((0,)), Wn, np.zeros(5), 0, 0)
    assert np.allclose(qt, oracle.absorb(q, Wn), rtol=1e-14, atol=1e-14)
    assert np.array_equal(b, np.zeros((2, 3)))
    C = rng.standard_normal((9, 7))
    w = rng.random(3)
    e1 = oracle.score_explicit_rope(q[0], np.zeros((0,)), Wn, np.zeros(5), w, C, np.arange(9), 0, 0)
    e2 = oracle.score_explicit(q[0], Wn, w, C)
    assert np.allclose(e1, e2, rtol=1e-13, atol=1e-13)


def pin_worked_bias_before_relu():
    g = _golden("worked_rope.json")["bias_relu"]
    for bias, want in g["cases"]:
        got = oracle.score(np.array(g["qt"]), np.array(g["w"]), np.array(g["c"]), bias=np.array([bias]))
        assert got[0] == want, (bias, got)


def pin_bias_is_an_extra_latent_column():
    rng = np.random.default_rng(24)
    H, r, n = 4, 9, 30
    qt = rng.standard_normal((H, r))
    b = rng.standard_normal(H) * 2.0
    w = rng.random(H)
    C = rng.standard_normal((n, r))
    s1 = oracle.score(qt, w, C, bias=b)
    s2 = oracle.score(np.concatenate([qt, b[:, None]], axis=1), w, np.concatenate([C, np.ones((n, 1))], axis=1))
    assert np.array_equal(s1, s2)
    assert np.any(s1 != oracle.score(qt, w, C))


def pin_fp8_score_with_bias_is_plain_score_of_dequantized_rows():
    rng = np.random.default_rng(25)
    H, r, n = 5, 256, 40
    qc, qs = oracle.quantize_rows(rng.standard_normal((H, r)).astype(np.float32))
    cc, cs = oracle.quantize_rows(rng.standard_normal((n, r)).astype(np.float32))
    b = rng.standard_normal(H) * 3.0
    w = rng.random(H)
    deq = lambda c, s: oracle.e4m3_decode(c) * np.repeat(s.astype(np.float64), 128, axis=-1)
    want = oracle.score(deq(qc, qs), w, deq(cc, cs), bias=b)
    got = oracle.score_fp8(qc, qs, w, cc, cs, bias=b)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]

"""GPU: the whole-model indexer composition (sparse_attention_token_absorb_amd.model)
against the oracle, layer by layer, with the rows each layer scored counted.

Layer maps and methods follow the LatentIndex summary page (§C.3: an
independent first layer, then groups; §3.2/§C.4: hierarchical selection;
§3.4/§B.3: the number of scored positions).  Every layer's selection is held
to the usual parity rules (tests/parity.py).  The rows a layer scored are
read off its score buffer: every buffer is filled with NaN before the step,
the library writes exactly the scores of the rows it scored and leaves the
rest untouched, so the finite entries are the scored rows; their sums are
compared with the oracle's closed forms.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from parity import check_scores, check_topk, rms
from sparse_attention_token_absorb_amd import binding as B
from sparse_attention_token_absorb_amd import synth
from sparse_attention_token_absorb_amd.model import IndexerModel, LayerMap

pytestmark = pytest.mark.gpu


def say(msg: str) -> None:
    print(f"[model] {msg}", flush=True)
    sys.stdout.flush()


def _gpu():
    import gpu_harness
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    return gpu_harness


def _fp8_cache(h, g, rows, r):
    dev = h.device()
    pool = torch.zeros((max(g.num_pages, 1), 64, r), dtype=torch.uint8, device=dev)
    scales = torch.zeros((max(g.num_pages, 1), 64, r // 128), dtype=torch.float32, device=dev)
    cache = B.LatentCache(pool, h.i32(g.block_table), h.i32(g.lens), scales)
    for b in range(g.B):
        n = int(g.lens[b])
        B.append_latent(cache, h.to_dev(rows[b][:n], torch.bfloat16), h.i32(np.full(n, b)), h.i32(np.arange(n)))
    return cache


def _model(h, g, lmap, fp8=False, keep_scores=True, M=None):
    """Key caches hold each layer's decoder applied to the latent; every
    group's latent cache holds the same latent rows (written by appends)."""
    keys, lats = {}, []
    for l in range(lmap.n_layers):
        keys[l] = _fp8_cache(h, g, g.keys_a[l], g.d) if fp8 else h.build_cache(g, latent=g.keys_a[l], r=g.d)
    for _ in lmap.groups:
        lats.append(_fp8_cache(h, g, g.latent, g.r) if fp8 else h.build_cache(g))
    bf = torch.bfloat16
    q = [h.to_dev(g.q[l], bf) for l in range(lmap.n_layers)]
    W = [h.to_dev(g.W[l], bf) for l in range(lmap.n_layers)]
    w = [h.head_weights(g, l) for l in range(lmap.n_layers)]
    qs = h.Queries(g)
    m = IndexerModel(lmap, keys, lats, q, W, w, g.k, g.M if M is None else M, qs.max_valid, fp8=fp8,
                     keep_scores=keep_scores)
    return m, qs


def _poison(m):
    for o in m.out + m.out_anchor + m.out_follower:
        if o.scores is not None:
            o.scores.fill_(float("nan"))


def _finite_rows(t):
    """Per query: the number of finite entries, and whether they form a prefix."""
    f = torch.isfinite(t).cpu().numpy()
    counts = f.sum(axis=1)
    prefix = all(f[i, :c].all() for i, c in enumerate(counts))
    return counts, prefix


# ----------------------------------------------------------------------------
# Oracle views of one layer (bf16 path: the oracle sees the stored bf16 values;
# FP8 path: the oracle quantizes the same bf16 rows and queries itself)
# ----------------------------------------------------------------------------
class OracleModel:
    def __init__(self, g, fp8):
        self.g, self.fp8 = g, fp8
        if fp8:
            self.lat8 = [oracle.quantize_rows(g.latent[b][:int(g.lens[b])]) for b in range(g.B)]
            self._keys8 = {}

    def _n(self, i):
        g = self.g
        return oracle.valid_rows(g.qpos[i], g.lens[int(g.qseq[i])])

    def native(self, l, i):
        g = self.g
        b, n = int(g.qseq[i]), self._n(i)
        if not self.fp8:
            return oracle.score_explicit(g.q[l][i], None, g.w[l][i], g.keys_a[l][b], n)
        if l not in self._keys8:
            self._keys8[l] = [oracle.quantize_rows(g.keys_a[l][bb][:int(g.lens[bb])]) for bb in range(g.B)]
        qc, qsc = oracle.quantize_rows(g.q[l][i])
        cc, cs = self._keys8[l][b]
        return oracle.score_fp8(qc, qsc, g.w[l][i], cc, cs, n=n)

    def latent(self, l, i, rows=None):
        g = self.g
        b, n = int(g.qseq[i]), self._n(i)
        if not self.fp8:
            qt = oracle.absorb(g.q[l][i], g.W[l])
            return oracle.score(qt, g.w[l][i], g.latent[b], n=None if rows is not None else n, rows=rows)
        qc, qsc = oracle.absorb_fp8(g.q[l][i][None], g.W[l])
        cc, cs = self.lat8[b]
        return oracle.score_fp8(qc[0], qsc[0], g.w[l][i], cc, cs, n=None if rows is not None else n, rows=rows)


def _check_full(o, sel, scores, i, K, tag):
    gi, gc = sel.idx.cpu().numpy(), sel.count.cpu().numpy()
    if scores is not None:
        check_scores(scores[i, :len(o)], o, f"{tag} scores")
    check_topk(gi[i], int(gc[i]), oracle.topk(o, K), o, None, K, rms(o), f"{tag} top-{K}")


def _verify(m, g, om, method, sel):
    """Every layer's selection under `method` against the oracle."""
    k, M = m.k, m.M
    for i in range(g.Q):
        n = om._n(i)
        K = min(k, n)
        for l in m.lmap.independent:
            o = om.native(l, i)
            sc = m.out[l].scores.cpu().numpy() if m.out[l].scores is not None else None
            _check_full(o, sel[l], sc, i, K, f"{method} independent layer {l} q{i}")
        for gi, layers in enumerate(m.lmap.groups):
            a = layers[0]
            if method in ("dsa", "indexcache"):
                for l in (layers if method == "dsa" else layers[:1]):
                    o = om.native(l, i)
                    sc = m.out[l].scores.cpu().numpy() if m.out[l].scores is not None else None
                    _check_full(o, sel[l], sc, i, K, f"{method} layer {l} q{i}")
                if method == "indexcache":
                    for l in layers[1:]:
                        assert sel[l] is sel[a], "index reuse: followers take the anchor's selection"
                continue
            if method == "latentindex":
                for l in layers:
                    o = om.latent(l, i)
                    sc = m.out[l].scores.cpu().numpy() if m.out[l].scores is not None else None
                    _check_full(o, sel[l], sc, i, K, f"{method} layer {l} q{i}")
                continue
            # hs: anchor candidates and nested selection, then followers inside the candidates
            s0 = om.latent(a, i)
            rho0 = rms(s0)
            Me = min(M, n)
            ca = m.candidates(gi)
            cidx, ccnt = ca.idx.cpu().numpy(), ca.count.cpu().numpy()
            check_topk(cidx[i], int(ccnt[i]), oracle.topk(s0, Me), s0, None, Me, rho0, f"hs group {gi} cand q{i}")
            cand = cidx[i, :Me].astype(np.int64)
            Ke = min(k, Me)
            inner = sel[a]
            check_topk(inner.idx.cpu().numpy()[i], int(inner.count.cpu().numpy()[i]),
                       oracle.topk(s0[cand], Ke, pos=cand), {int(p): s0[p] for p in cand}, cand, Ke, rho0,
                       f"hs group {gi} anchor top-k q{i}")
            for l in layers[1:]:
                cs = om.latent(l, i, rows=cand.astype(np.int32))
                fo = sel[l]
                if fo.scores is not None:
                    check_scores(fo.scores.cpu().numpy()[i, :Me], cs, f"hs follower {l} q{i} scores")
                check_topk(fo.idx.cpu().numpy()[i], int(fo.count.cpu().numpy()[i]), oracle.topk(cs, Ke, pos=cand),
                           dict(zip(cand.tolist(), cs)), cand, Ke, rms(cs), f"hs follower {l} q{i} top-k")


def _rows_scored(m, method, sel):
    """Rows scored per query: (per independent layer, per group) from the
    finite entries of the score buffers."""
    per_group = []
    ind = []
    for l in m.lmap.independent:
        c, prefix = _finite_rows(m.out[l].scores)
        assert prefix
        ind.append(c)
    for gi, layers in enumerate(m.lmap.groups):
        tot = 0
        for j, l in enumerate(layers):
            if method == "indexcache" and j > 0:
                continue  # reuse: nothing scored
            if method == "hs" and j == 0:
                t = m.out_anchor[gi].scores
            elif method == "hs":
                t = m.out_follower[l].scores
            else:
                t = m.out[l].scores
            c, prefix = _finite_rows(t)
            assert prefix, f"{method} layer {l}: scored entries are not a prefix of the buffer"
            tot = tot + c
        per_group.append(tot)
    return ind, per_group


# ----------------------------------------------------------------------------
# Tests
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_group_of_eight_every_method(fp8):
    """One group of 8 layers (anchor + 7 followers) on two ragged sequences:
    each method's selections against the oracle, and the rows scored per
    group against the closed forms n G (full) and n + (G-1) min(M, n) (HS)."""
    h = _gpu()
    g = synth.make_decode("model8", 81, B=2, lens=[3000, 1700], r=256, H=64, d=128, k=256, M=1024, G=8,
                          keys_a=True)
    lmap = LayerMap(8, (), (tuple(range(8)),))
    m, qs = _model(h, g, lmap, fp8=fp8)
    om = OracleModel(g, fp8)
    n = np.array([om._n(i) for i in range(g.Q)])
    for method in ("latentindex", "hs", "dsa", "indexcache"):
        say(f"group of 8 ({'fp8' if fp8 else 'bf16'}): {method}")
        _poison(m)
        sel = m.step(method, qs.seq, qs.pos)
        torch.cuda.synchronize()
        _verify(m, g, om, method, sel)
        _, groups = _rows_scored(m, method, sel)
        got = groups[0]
        if method == "hs":
            want = [oracle.rows_scored_hs(int(x), min(g.M, int(x)), 8) for x in n]
        elif method == "indexcache":
            want = [int(x) for x in n]
        else:
            want = [oracle.rows_scored_full(int(x), 8) for x in n]
        assert list(got) == want, (method, list(got), want)
        say(f"{method}: rows scored per query {list(got)}")


def test_index_reuse_budget_equals_hs_with_m_equal_k():
    """HS with M = k: every follower returns the anchor's candidate set."""
    h = _gpu()
    g = synth.make_decode("model-reuse", 82, B=2, lens=[5000, 900], r=256, H=64, d=128, k=512, M=512, G=4,
                          keys_a=True)
    lmap = LayerMap(4, (), ((0, 1, 2, 3),))
    m, qs = _model(h, g, lmap, keep_scores=False)
    sel = m.step("hs", qs.seq, qs.pos)
    torch.cuda.synchronize()
    cand = m.candidates(0).idx.cpu().numpy()
    for l in (1, 2, 3):
        fi = sel[l].idx.cpu().numpy()
        for i in range(g.Q):
            assert set(fi[i].tolist()) == set(cand[i].tolist())


def test_small_model_maps_and_scored_positions():
    """Layer 0 on its own, then a group of 8 and a group of 4 (the pages' G = 8
    map at small scale), and a uniform G = 4 map; every layer against the
    oracle, and the rows scored by the whole model against the closed form
    independent L + groups (L + (G-1) min(M, L))."""
    h = _gpu()
    g = synth.make_decode("model13", 83, B=2, lens=[2600, 1400], r=256, H=32, d=128, k=128, M=512, G=13,
                          keys_a=True)
    om = OracleModel(g, False)
    n = np.array([om._n(i) for i in range(g.Q)])
    for lmap in (LayerMap.grouped(13, 8), LayerMap.grouped(9, 4)):
        say(f"map {lmap.group_sizes()}")
        m, qs = _model(h, g, lmap)
        for method in ("dsa", "latentindex", "hs", "indexcache"):
            _poison(m)
            sel = m.step(method, qs.seq, qs.pos)
            torch.cuda.synchronize()
            _verify(m, g, om, method, sel)
            ind, groups = _rows_scored(m, method, sel)
            total = sum(ind) + sum(groups)
            if method == "hs":
                want = [int(x) * len(lmap.independent) +
                        sum(oracle.rows_scored_hs(int(x), min(g.M, int(x)), G) for G in lmap.group_sizes()) for x in n]
                if len(set(lmap.group_sizes())) == 1:
                    G = lmap.group_sizes()[0]
                    assert want == [oracle.model_positions_hs(int(x), len(lmap.independent), len(lmap.groups), G, g.M)
                                    for x in n]
            elif method == "indexcache":
                want = [int(x) * (len(lmap.independent) + len(lmap.groups)) for x in n]
            else:
                want = [oracle.rows_scored_full(int(x), lmap.n_layers) for x in n]
            assert list(total) == want, (lmap.group_sizes(), method, list(total), want)
            say(f"map {lmap.group_sizes()} {method}: rows scored per query {list(total)}")
        del m
        torch.cuda.empty_cache()


def test_hs_with_budget_covering_every_row_runs_as_full_latentindex():
    """When max_valid <= M every candidate set is the whole prefix, so HS is
    full LatentIndex on the group (§3.2, §C.4): the step's selections equal
    the full method's and the oracle's, and no candidate list is claimed."""
    h = _gpu()
    g = synth.make_decode("model-covered", 84, B=2, lens=[1500, 900], r=256, H=64, d=128, k=256, M=2048, G=4,
                          keys_a=True)
    lmap = LayerMap(4, (), ((0, 1, 2, 3),))
    m, qs = _model(h, g, lmap)
    assert qs.max_valid <= g.M
    om = OracleModel(g, False)
    full = m.step("latentindex", qs.seq, qs.pos)
    torch.cuda.synchronize()
    want = {l: (full[l].idx.cpu().numpy().copy(), full[l].count.cpu().numpy().copy()) for l in range(4)}
    _poison(m)
    sel = m.step("hs", qs.seq, qs.pos)
    torch.cuda.synchronize()
    _verify(m, g, om, "latentindex", sel)
    for l in range(4):
        gi, gc = sel[l].idx.cpu().numpy(), sel[l].count.cpu().numpy()
        assert np.array_equal(gc, want[l][1])
        for i in range(g.Q):
            assert set(gi[i, :gc[i]].tolist()) == set(want[l][0][i, :gc[i]].tolist()), (l, i)
    with pytest.raises(ValueError):
        m.candidates(0)
    _, groups = _rows_scored(m, "latentindex", sel)
    n = [om._n(i) for i in range(g.Q)]
    assert list(groups[0]) == [oracle.rows_scored_hs(x, min(g.M, x), 4) for x in n]

"""Selection checked exactly against the GPU's own scores.

The parity tests compare selections with the oracle's under a score
tolerance.  These cases pin the selection itself: with the scores the
kernels kept (``keep_scores``), every call's output must be an exact top-K
of them (LatentIndex, paperlayer.ai summary of arXiv:2610.04635, §3.1 and
§4.1 for the per-layer top-k, §3.2 for the anchor's top-M with its nested
top-k and the followers' top-k among the candidates): K = min(n, k) distinct
positions, padding -1, and no unselected row scoring above a selected one.
Rows are drawn from a small set of distinct rows, so many scores are exactly
equal; every tie-breaking path of the radix selection runs (long equal
runs, threshold digits of at most 64 elements, sign-spanning keys, the
streaming and many-workgroup modes, the nested selection over the outer
winners).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from sparse_attention_token_absorb_amd import binding as B
from sparse_attention_token_absorb_amd.synth import round_bf16

pytestmark = pytest.mark.gpu

R, H = 256, 64


def _dev():
    return torch.device("cuda:0")


def _i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(_dev())


def _setup(seed, lens, distinct, w_sign=False, Q_per_seq=1):
    """Cache of len(lens) sequences whose rows repeat `distinct` random rows;
    Q_per_seq queries per sequence at its last position."""
    rng = np.random.default_rng(seed)
    lens = [int(n) for n in lens]
    pages = [(n + 63) // 64 for n in lens]
    maxp = max(pages)
    bt = np.full((len(lens), maxp), -1, dtype=np.int32)
    perm = rng.permutation(sum(pages)).astype(np.int32)
    o = 0
    for b, p in enumerate(pages):
        bt[b, :p] = perm[o:o + p]
        o += p
    pool = torch.zeros((max(sum(pages), 1), 64, R), dtype=torch.bfloat16, device=_dev())
    cache = B.LatentCache(pool, _i32(bt), _i32(lens))
    base = round_bf16(rng.standard_normal((distinct, R), dtype=np.float32))
    for b, n in enumerate(lens):
        rows = base[rng.integers(0, distinct, size=n)]
        B.append_latent(cache, torch.from_numpy(rows).to(torch.bfloat16).to(_dev()), _i32(np.full(n, b)),
                        _i32(np.arange(n)))
    qseq = np.repeat(np.arange(len(lens)), Q_per_seq).astype(np.int32)
    qpos = np.array([lens[s] - 1 for s in qseq], dtype=np.int32)
    Q = len(qseq)
    qt = torch.from_numpy(round_bf16(rng.standard_normal((Q, H, R), dtype=np.float32) * np.float32(0.1)))
    w = rng.random((Q, H), dtype=np.float32) + np.float32(0.05)
    if w_sign:
        w *= np.where(rng.random((Q, H)) < 0.5, -1.0, 1.0).astype(np.float32)
    n_q = [lens[s] for s in qseq]
    return (cache, _i32(qseq), _i32(qpos), max(n_q), qt.to(torch.bfloat16).to(_dev()),
            torch.from_numpy(w).to(_dev()), n_q)


def _host(t):
    return t.detach().cpu().numpy()


def assert_exact_topk(scores, sel, count, K, what):
    """sel[:K] is an exact top-K of `scores` (indices into it), -1 after."""
    assert int(count) == K, f"{what}: count {int(count)} != {K}"
    s = np.asarray(sel[:K], dtype=np.int64)
    assert np.all(np.asarray(sel[K:]) == -1), f"{what}: padding is not -1"
    assert len(np.unique(s)) == K, f"{what}: duplicates"
    assert K == 0 or (s.min() >= 0 and s.max() < scores.size), f"{what}: index outside the row"
    if K == 0 or K == scores.size:
        return
    rest = np.ones(scores.size, dtype=bool)
    rest[s] = False
    lo, hi = scores[s].min(), scores[rest].max()
    assert lo >= hi, f"{what}: selected minimum {lo!r} below unselected maximum {hi!r}"


def _check_full(out, n_q, k, what, k_inner=0):
    idx, cnt, sc = _host(out.idx), _host(out.count), _host(out.scores)
    for i, n in enumerate(n_q):
        assert_exact_topk(sc[i, :n], idx[i], cnt[i], min(n, k), f"{what} q{i}")
        if k_inner:
            inner = _host(out.idx_inner)[i]
            Ki = min(n, k_inner)
            assert_exact_topk(sc[i, :n], inner, _host(out.count_inner)[i], Ki, f"{what} inner q{i}")
            assert set(inner[:Ki].tolist()) <= set(idx[i, :min(n, k)].tolist()), f"{what} q{i}: inner not nested"


@pytest.mark.parametrize("lens,distinct,k", [
    ([40, 64, 65], 1, 16),            # one distinct row: every score equal
    ([300, 64, 1], 7, 50),            # short rows, long equal runs
    ([8192], 30, 2048),               # ~270 copies per value: equal run across all digits
    ([8192, 5000], 200, 2048),        # ~40 copies per value: threshold digit of <= 64 equal keys
    ([8192, 8191, 4097], 8192, 2048),  # mostly distinct: a few elements left after the first digit
    ([40, 64, 65, 8192], 50, 8192),   # the budget covers every row: all taken without a radix pass
])
def test_short_rows_exact(lens, distinct, k):
    cache, seq, pos, mv, qt, w, n_q = _setup(11 + distinct, lens, distinct)
    out = B.score_topk(cache, seq, pos, mv, qt, w, k, keep_scores=True)
    _check_full(out, n_q, k, f"lens={lens} distinct={distinct}")


@pytest.mark.parametrize("lens,distinct,k", [
    ([16384, 12000, 8193], 1, 2048),     # every score equal: a tie list as long as the longest row
    ([16384, 9000], 30, 2048),           # long equal runs
    ([16384, 16000, 10000], 16384, 2048),  # mostly distinct
    ([16384, 12000], 40, 16384),         # the budget covers every row
])
def test_rows_up_to_16384_exact(lens, distinct, k):
    # a few queries over rows of 8193..16384 scores: one workgroup per query
    # holds all of a row's keys and counts them itself (no histogram from the
    # scoring kernel)
    cache, seq, pos, mv, qt, w, n_q = _setup(61 + distinct, lens, distinct)
    out = B.score_topk(cache, seq, pos, mv, qt, w, k, keep_scores=True)
    _check_full(out, n_q, k, f"lens={lens} distinct={distinct}")


def test_sign_spanning_scores_exact():
    cache, seq, pos, mv, qt, w, n_q = _setup(5, [3000, 2500], 500, w_sign=True)
    out = B.score_topk(cache, seq, pos, mv, qt, w, 700, keep_scores=True)
    sc = _host(out.scores)
    assert (sc[0, :3000] < 0).any() and (sc[0, :3000] > 0).any()
    _check_full(out, n_q, 700, "signed")


@pytest.mark.parametrize("distinct", [3, 500, 40000])
def test_long_rows_exact(distinct):
    # rows beyond 16384 with few queries: the many-workgroup filter and the
    # final kernel (3 distinct rows: tie lists beyond the LDS list)
    cache, seq, pos, mv, qt, w, n_q = _setup(21, [40000, 23000], distinct)
    out = B.score_topk(cache, seq, pos, mv, qt, w, 2048, k_inner=512, keep_scores=True)
    _check_full(out, n_q, 2048, f"long distinct={distinct}", k_inner=512)


@pytest.mark.parametrize("mode", [B.FUSED_FILTER_OFF, B.FUSED_FILTER_FALLBACK])
@pytest.mark.parametrize("distinct", [3, 40000])
def test_long_rows_exact_in_every_filter_mode(mode, distinct):
    # the filter pass in a kernel of its own, and the fused pass whose wait
    # runs out at once (every query then selected again by the final kernel
    # from its scores alone, the nested selection over the outer winners)
    B.fused_filter(mode)
    try:
        cache, seq, pos, mv, qt, w, n_q = _setup(21, [40000, 23000], distinct)
        out = B.score_topk(cache, seq, pos, mv, qt, w, 2048, k_inner=512, keep_scores=True)
        _check_full(out, n_q, 2048, f"long distinct={distinct} mode={mode}", k_inner=512)
        out = B.score_topk(cache, seq, pos, mv, qt, w, 5000, keep_scores=True)
        _check_full(out, n_q, 5000, f"long k=5000 distinct={distinct} mode={mode}")
    finally:
        B.fused_filter(B.FUSED_FILTER_ON)


@pytest.mark.parametrize("fill", ["random", "ones"])
@pytest.mark.parametrize("mode", [B.FUSED_FILTER_ON, B.FUSED_FILTER_OFF])
def test_long_rows_with_a_dirty_workspace(mode, fill):
    # a workspace that was not zero-filled: the filter path cannot trust the
    # histogram in its leading region (the bins do not sum to the row count)
    # nor a published threshold word (all ones sets its flag but names no
    # query's row count), the final kernel selects again from the scores, and
    # every call leaves the region zeroed, so the calls after it run the
    # normal path
    B.fused_filter(mode)
    try:
        cache, seq, pos, mv, qt, w, n_q = _setup(23, [40000, 23000], 500)
        nb = B.workspace_bytes(B.LI_OP_SCORE_TOPK, len(n_q), mv, H, R, 2048, 0)
        if fill == "random":
            ws = torch.randint(0, 256, (nb,), dtype=torch.uint8, device=_dev())
        else:
            ws = torch.full((nb,), 255, dtype=torch.uint8, device=_dev())
        for rep in range(3):
            out = B.score_topk(cache, seq, pos, mv, qt, w, 2048, k_inner=512, keep_scores=True, ws=ws)
            _check_full(out, n_q, 2048, f"dirty workspace, call {rep}, mode {mode}", k_inner=512)
    finally:
        B.fused_filter(B.FUSED_FILTER_ON)


# The zeroed region's per-query record (internal layout, read only by the
# test below): 4096 first-digit bins, then counters; the tenth counter is the
# number of rows the fused filter pass has sorted.
_REC_INTS = 4096 + 16
_SLOT_DONE = 4096 + 9


@pytest.mark.parametrize("k_inner", [0, 512])
def test_mixed_lengths_finish_inside_the_scoring_launch(k_inner):
    # queries of different lengths in one batch: the workgroups past a short
    # query's last row hold no rows and take no part in its filter pass, so
    # each query's rows are all sorted inside the scoring launch (its count
    # of sorted rows reaches n) and the final kernel does not select again
    # from the scores; before, their empty row counts kept the row total
    # from ever meeting n, and every short query waited out its bound
    lens = [65536, 40000, 23000, 17000]
    cache, seq, pos, mv, qt, w, n_q = _setup(27 + k_inner, lens, 500)
    nb = B.workspace_bytes(B.LI_OP_SCORE_TOPK_EXT_SCORES, len(n_q), mv, H, R, 2048, 0)
    ws = B.workspace(nb, _dev())
    for rep in range(2):
        out = B.score_topk(cache, seq, pos, mv, qt, w, 2048, k_inner=k_inner, keep_scores=True, ws=ws)
        _check_full(out, n_q, 2048, f"mixed lengths, call {rep}", k_inner=k_inner)
        torch.cuda.synchronize()
        rec = ws[: len(n_q) * _REC_INTS * 4].view(torch.int32).view(len(n_q), _REC_INTS).cpu().numpy()
        done = rec[:, _SLOT_DONE].tolist()
        assert done == [int(n) for n in n_q], f"call {rep}: rows sorted by the filter pass {done}, rows {n_q}"


def test_concurrent_launches_on_two_streams_stay_exact():
    # two long-row calls enqueued on two streams at once, each with a grid
    # that fills the GPU: the fused filter pass of one may find its
    # workgroups not all resident while the other holds CUs (a bounded wait,
    # then the final kernel's reselection from the scores); every result
    # must still be an exact top-k with its nested top-k
    cache, seq, pos, mv, qt, w, n_q = _setup(29, [65536, 65536, 65536, 65536], 3000)
    qt2 = (qt.float() * -1.0).to(torch.bfloat16)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    torch.cuda.synchronize()
    for rep in range(3):
        for si, (st, q_) in enumerate(zip(streams, (qt, qt2))):
            with torch.cuda.stream(st):
                outs.append((rep, si, B.score_topk(cache, seq, pos, mv, q_, w, 2048, k_inner=512, keep_scores=True)))
    torch.cuda.synchronize()
    for rep, si, out in outs:
        _check_full(out, n_q, 2048, f"concurrent call {rep} on stream {si}", k_inner=512)


def test_many_queries_stream_exact():
    # more than 64 queries over rows beyond 8192: the streaming selection
    cache, seq, pos, mv, qt, w, n_q = _setup(31, [12000, 9000, 20000], 60, Q_per_seq=24)
    out = B.score_topk(cache, seq, pos, mv, qt, w, 2048, keep_scores=True)
    _check_full(out, n_q, 2048, "stream")


@pytest.mark.parametrize("lens,distinct,M,k", [
    ([5000, 3000], 100, 2048, 512),    # short anchor rows: nested selection over the outer winners
    ([20000, 30000], 100, 8192, 2048),  # long anchor rows: nested selection in the filter
    ([20000, 900], 9, 8192, 2048),     # a sequence shorter than M, massive ties
    ([5000, 3000, 8192], 40, 8192, 2048),  # M covers every row: the anchor keeps all, its top-k nested
    ([16384, 12000], 60, 8192, 2048),  # anchor rows of up to 16384: the one-workgroup selection counts them
])
def test_hs_exact(lens, distinct, M, k):
    cache, seq, pos, mv, qt, w, n_q = _setup(41 + M, lens, distinct)
    anchor = B.score_topk(cache, seq, pos, mv, qt, w, M, k_inner=k, keep_scores=True)
    _check_full(anchor, n_q, M, "anchor", k_inner=k)
    rng = np.random.default_rng(7)
    qt2 = torch.from_numpy(round_bf16(rng.standard_normal(tuple(qt.shape), dtype=np.float32) * np.float32(0.1)))
    fol = B.hs_select(cache, seq, pos, mv, anchor.idx, anchor.count, qt2.to(torch.bfloat16).to(_dev()), w, k,
                      keep_scores=True)
    a_idx, a_cnt = _host(anchor.idx), _host(anchor.count)
    f_idx, f_cnt, f_sc = _host(fol.idx), _host(fol.count), _host(fol.scores)
    for i, n in enumerate(n_q):
        c = int(a_cnt[i])
        cand = a_idx[i, :c]
        pos_of = {int(p): j for j, p in enumerate(cand)}
        K = min(c, k)
        sel = f_idx[i]
        assert np.all(sel[K:] == -1), f"follower q{i}: padding is not -1"
        assert set(sel[:K].tolist()) <= set(pos_of), f"follower q{i}: selected outside the candidates"
        local = np.array([pos_of[int(p)] for p in sel[:K]] + [-1] * (k - K), dtype=np.int64)
        assert_exact_topk(f_sc[i, :c], local, f_cnt[i], K, f"follower q{i}")

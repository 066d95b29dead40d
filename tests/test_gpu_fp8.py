"""GPU parity of the segmented FP8 path against the oracle (needs an MI355X).

The latent rows enter as bf16 values, so the GPU's rotation and quantization
see exactly the oracle's inputs and must reproduce its codes and scales bit
for bit.  The absorbed query is summed in fp64 on both sides (exact for bf16
data) and rounded once to fp32, so its codes and scales must match bit for
bit too.  Scores and top-k sets follow the same rules as the bf16 path
(tests/parity.py), both sides scoring the same quantized operands.
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

pytestmark = pytest.mark.gpu


def say(msg: str) -> None:
    print(f"[fp8] {msg}", flush=True)
    sys.stdout.flush()


def _gpu():
    import gpu_harness
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    return gpu_harness


def fp8_cache(h, g, r=None):
    """Page pool of codes + scales, rows written through li_append_latent."""
    dev = h.device()
    r = g.r if r is None else r
    pool = torch.zeros((max(g.num_pages, 1), 64, r), dtype=torch.uint8, device=dev)
    scales = torch.zeros((max(g.num_pages, 1), 64, r // 128), dtype=torch.float32, device=dev)
    cache = B.LatentCache(pool, h.i32(g.block_table), h.i32(g.lens), scales)
    for b in range(g.B):
        n = int(g.lens[b])
        if n:
            B.append_latent(cache, h.to_dev(g.latent[b][:n], torch.bfloat16), h.i32(np.full(n, b)), h.i32(np.arange(n)))
    return cache


def slot_of(g, b, j):
    return int(g.block_table[b][j // 64]) * 64 + j % 64


def oracle_codes(g):
    return [oracle.quantize_rows(g.latent[b][: int(g.lens[b])]) for b in range(g.B)]


def test_fp8_append_is_bit_exact():
    h = _gpu()
    for r in (256, 128):
        say(f"append r={r}")
        g = synth.make_decode("f8app", 60 + r, B=3, lens=[700, 130, 64], r=r, H=8, d=64, k=64, M=128)
        g.latent[0][5] = 0.0                                      # all-zero row: scale 1, codes 0
        g.latent[0][6] = synth.round_bf16(g.latent[0][6] * 3e4)   # large magnitudes
        g.latent[0][7] = synth.round_bf16(g.latent[0][7] * 1e-30)  # tiny magnitudes
        g.latent[1][9, :] = synth.round_bf16(np.float32(2.0) ** -20)
        cache = fp8_cache(h, g, r)
        pool = h.host(cache.pool).reshape(-1, r)
        sc = h.host(cache.scales).reshape(-1, r // 128)
        for b, (codes, scales) in enumerate(oracle_codes(g)):
            slots = [slot_of(g, b, j) for j in range(int(g.lens[b]))]
            assert np.array_equal(pool[slots], codes), f"r={r} seq {b}: codes differ"
            assert np.array_equal(sc[slots], scales), f"r={r} seq {b}: scales differ"


def test_fp8_absorb_is_bit_exact():
    h = _gpu()
    # row counts that take each of the three row-block sizes, every d
    for (Q, H, d, r) in ((3, 64, 128, 256), (5, 7, 64, 128), (2, 33, 256, 256), (40, 64, 128, 256),
                         (530, 64, 32, 128)):
        say(f"absorb Q={Q} H={H} d={d} r={r}")
        rng = np.random.default_rng(Q * 100 + H)
        q = synth.round_bf16(rng.standard_normal((Q, H, d)).astype(np.float32))
        W = synth.round_bf16((rng.standard_normal((d, r)) / np.sqrt(r)).astype(np.float32))
        q[0, 0] = 0.0                                          # an all-zero query row
        fq = B.absorb_query(h.to_dev(q, torch.bfloat16), h.to_dev(W, torch.bfloat16), fp8=True)
        gc, gs = h.host(fq.codes()), h.host(fq.scales())
        oc, os_ = oracle.absorb_fp8(q, W)
        assert np.array_equal(gs, os_), f"scales differ at {np.argwhere(gs != os_)[:4].tolist()}"
        assert np.array_equal(gc, oc), f"codes differ at {np.argwhere(gc != oc)[:4].tolist()}"


def test_fp8_query_without_decoder_is_bit_exact():
    """No decoder (a per-layer indexer's own query): q itself is rotated and
    quantized, bit for bit what the oracle gives for an identity decoder, at
    every row-block size."""
    h = _gpu()
    for (Q, H, r) in ((1, 64, 128), (3, 64, 256), (40, 64, 128), (530, 64, 256)):
        say(f"no-decoder quantization Q={Q} H={H} r={r}")
        rng = np.random.default_rng(700 + Q + r)
        q = synth.round_bf16(rng.standard_normal((Q, H, r)).astype(np.float32))
        q[0, 0] = 0.0
        q[-1, -1, :7] = synth.round_bf16(np.float32(3e4))
        fq = B.absorb_query(h.to_dev(q, torch.bfloat16), None, fp8=True)
        gc, gs = h.host(fq.codes()), h.host(fq.scales())
        oc, os_ = oracle.absorb_fp8(q, np.eye(r, dtype=np.float32))
        assert np.array_equal(gs, os_), f"scales differ at {np.argwhere(gs != os_)[:4].tolist()}"
        assert np.array_equal(gc, oc), f"codes differ at {np.argwhere(gc != oc)[:4].tolist()}"


def fp8_layer(h, g, cache, qs, l, k=None, k_inner=0):
    fq = B.absorb_query(h.to_dev(g.q[l], torch.bfloat16), h.to_dev(g.W[l], torch.bfloat16), fp8=True)
    out = B.score_topk(cache, qs.seq, qs.pos, qs.max_valid, fq, h.head_weights(g, l), g.k if k is None else k,
                       k_inner=k_inner, keep_scores=True)
    return fq, out


def verify_fp8_full(h, g, l, out, k=None, codes=None, tag="", queries=None):
    k = g.k if k is None else k
    codes = oracle_codes(g) if codes is None else codes
    oq, oqs = oracle.absorb_fp8(g.q[l], g.W[l])
    sel, cnt, sc = h.host(out.idx), h.host(out.count), h.host(out.scores)
    for i in (range(g.Q) if queries is None else queries):
        b = int(g.qseq[i])
        n = oracle.valid_rows(g.qpos[i], g.lens[b])
        cc, cs = codes[b]
        o = oracle.score_fp8(oq[i], oqs[i], g.w[l][i], cc, cs, n=n)
        check_scores(sc[i, :n], o, f"{tag} layer {l} query {i} scores")
        check_topk(sel[i], int(cnt[i]), oracle.topk(o, min(k, n)), o, None, min(k, n), rms(o),
                   f"{tag} layer {l} query {i} top-{k}")


def test_fp8_decode_8k_full_layers():
    h = _gpu()
    say("fp8 decode 8K, 4 layers")
    g = synth.decode_b1_n8192()
    cache = fp8_cache(h, g)
    qs = h.Queries(g)
    codes = oracle_codes(g)
    for l in range(g.G):
        _, out = fp8_layer(h, g, cache, qs, l)
        verify_fp8_full(h, g, l, out, codes=codes, tag="fp8-8k")


def verify_fp8_hs(h, g, cache, qs, codes, tag):
    """The anchor's top-M with its own top-k nested, then every follower
    rescoring the anchor's candidates, against the oracle on the same codes."""
    fq0, anchor = fp8_layer(h, g, cache, qs, 0, k=g.M, k_inner=g.k)
    a_idx, a_cnt = h.host(anchor.idx), h.host(anchor.count)
    a_in, a_in_cnt = h.host(anchor.idx_inner), h.host(anchor.count_inner)
    oq0, oqs0 = oracle.absorb_fp8(g.q[0], g.W[0])
    for l in range(1, g.G):
        fq = B.absorb_query(h.to_dev(g.q[l], torch.bfloat16), h.to_dev(g.W[l], torch.bfloat16), fp8=True)
        fo = B.hs_select(cache, qs.seq, qs.pos, qs.max_valid, anchor.idx, anchor.count, fq, h.head_weights(g, l), g.k,
                         keep_scores=True)
        oq, oqs = oracle.absorb_fp8(g.q[l], g.W[l])
        fi, fc, fs = h.host(fo.idx), h.host(fo.count), h.host(fo.scores)
        for i in range(g.Q):
            b = int(g.qseq[i])
            n = oracle.valid_rows(g.qpos[i], g.lens[b])
            Me, Ke = min(g.M, n), min(g.k, min(g.M, n))
            cc, cs = codes[b]
            if l == 1:
                s0 = oracle.score_fp8(oq0[i], oqs0[i], g.w[0][i], cc, cs, n=n)
                check_topk(a_idx[i], int(a_cnt[i]), oracle.topk(s0, Me), s0, None, Me, rms(s0), f"{tag} anchor q{i}")
                cand = a_idx[i, :Me].astype(np.int64)
                sub = {int(p): s0[p] for p in cand}
                check_topk(a_in[i], int(a_in_cnt[i]), oracle.topk(s0[cand], Ke, pos=cand), sub, cand, Ke, rms(s0),
                           f"{tag} anchor nested q{i}")
            cand = a_idx[i, :Me].astype(np.int32)
            cs_l = oracle.score_fp8(oq[i], oqs[i], g.w[l][i], cc, cs, rows=cand)
            check_scores(fs[i, :Me], cs_l, f"{tag} follower {l} q{i} scores")
            check_topk(fi[i], int(fc[i]), oracle.topk(cs_l, Ke, pos=cand), dict(zip(cand.tolist(), cs_l)), cand, Ke,
                       rms(cs_l), f"{tag} follower {l} q{i} top-k")


def test_fp8_ragged_paged_full_and_hs():
    h = _gpu()
    say("fp8 ragged paged: full + HS")
    g = synth.make_decode("f8rag", 61, B=5, lens=(3000, 20000), r=256, H=64, d=128, k=1024, M=4096)
    cache = fp8_cache(h, g)
    qs = h.Queries(g)
    codes = oracle_codes(g)
    _, out = fp8_layer(h, g, cache, qs, 1)
    verify_fp8_full(h, g, 1, out, codes=codes, tag="fp8-rag")
    verify_fp8_hs(h, g, cache, qs, codes, "fp8-rag")


def test_fp8_mixed_lengths_finish_inside_the_scoring_launch():
    """Four sequences of different lengths on the FP8 cache: the workgroups
    past a short query's last row take no part in its fused filter pass, so
    every query's rows are sorted inside the scoring launch (the count of
    sorted rows in the workspace's zeroed region, whose per-query record is
    4096 first-digit bins and then 16 counters, the tenth of them that
    count, reaches n) and the scores and top-k match the oracle."""
    h = _gpu()
    say("fp8 mixed lengths: fused filter pass completes for every query")
    g = synth.make_decode("f8mix", 63, B=4, lens=[65536, 40000, 23000, 17000], r=256, H=64, d=128, k=2048,
                          M=8192)
    cache = fp8_cache(h, g)
    qs = h.Queries(g)
    fq = B.absorb_query(h.to_dev(g.q[0], torch.bfloat16), h.to_dev(g.W[0], torch.bfloat16), fp8=True)
    nb = B.workspace_bytes(B.LI_OP_SCORE_TOPK_EXT_SCORES, g.Q, qs.max_valid, 64, 256, g.k, 0)
    ws = B.workspace(nb, h.device())
    out = B.score_topk(cache, qs.seq, qs.pos, qs.max_valid, fq, h.head_weights(g, 0), g.k, keep_scores=True, ws=ws)
    torch.cuda.synchronize()
    rec = ws[: g.Q * 4112 * 4].view(torch.int32).view(g.Q, 4112).cpu().numpy()
    n_q = [oracle.valid_rows(g.qpos[i], g.lens[int(g.qseq[i])]) for i in range(g.Q)]
    assert rec[:, 4096 + 9].tolist() == [int(n) for n in n_q], f"rows sorted {rec[:, 4096 + 9].tolist()}, rows {n_q}"
    verify_fp8_full(h, g, 0, out, tag="fp8-mixed")
    del cache
    torch.cuda.empty_cache()


def test_fp8_long_context_b4_n131072_full_and_hs():
    """The long-context workload (4 sequences of 131072 rows) on the FP8
    cache, in the launch configuration the benchmark times: every layer's
    full selection with every score, then the HS group (top-8192 anchor, 3
    followers)."""
    h = _gpu()
    g = synth.long_context_b4()
    say("fp8 long context B=4 N=131072: cache")
    cache = fp8_cache(h, g)
    qs = h.Queries(g)
    codes = oracle_codes(g)
    for l in range(g.G):
        say(f"fp8 long context full layer {l}")
        _, out = fp8_layer(h, g, cache, qs, l)
        verify_fp8_full(h, g, l, out, codes=codes, tag="fp8-long")
    say("fp8 long context HS M=8192")
    verify_fp8_hs(h, g, cache, qs, codes, "fp8-long")
    del cache
    torch.cuda.empty_cache()


def test_fp8_short_empty_and_r128():
    h = _gpu()
    say("fp8 short/empty sequences, r=128, few heads")
    g = synth.make_decode("f8short", 62, B=4, lens=[1, 0, 33, 257], r=128, H=5, d=32, k=16, M=64)
    cache = fp8_cache(h, g)
    qs = h.Queries(g)
    _, out = fp8_layer(h, g, cache, qs, 0)
    verify_fp8_full(h, g, 0, out, tag="fp8-short")


def test_fp8_prefill_sampled_rows():
    """4096 queries of one 65536-row sequence: the many-query kernel."""
    h = _gpu()
    g = synth.chunked_prefill_q4096()
    say("fp8 prefill Q=4096 N=65536: cache")
    cache = fp8_cache(h, g)
    qs = h.Queries(g)
    codes = oracle_codes(g)
    sample = h.prefill_sample(g.Q)
    assert len(sample) == 64 and sample[0] == 0 and sample[-1] == g.Q - 1
    for l in range(g.G):
        say(f"fp8 prefill layer {l}")
        _, out = fp8_layer(h, g, cache, qs, l)
        verify_fp8_full(h, g, l, out, codes=codes, tag="fp8-prefill", queries=sample)
        exp = np.minimum(g.k, np.minimum(g.qpos + 1, g.lens[0]))
        assert np.array_equal(h.host(out.count), exp)
        del out
        torch.cuda.empty_cache()


@pytest.mark.parametrize("r,Hh", [(256, 64), (128, 20)])
def test_fp8_prefill_mixed_sequences(r, Hh):
    """Many-query workgroups whose queries sit in different sequences, at
    scattered positions (causal prefixes of every length)."""
    h = _gpu()
    say(f"fp8 mixed-sequence prefill r={r} H={Hh}")
    g = synth.make_decode("f8mix", 63 + r, B=3, lens=[9000, 70, 5000], r=r, H=Hh, d=64, k=512, M=1024)
    Q = 52
    g.qseq = np.array([(i // 5) % 3 for i in range(Q)], dtype=np.int32)
    rng = np.random.default_rng(11)
    g.qpos = np.array([rng.integers(0, int(g.lens[b])) for b in g.qseq], dtype=np.int32)
    g.qpos[:3] = [0, 1, int(g.lens[0]) - 1]
    for l in range(2):
        g.q[l] = synth.round_bf16(np.random.default_rng(300 + l).standard_normal((Q, g.H, g.d)).astype(np.float32))
        g.w[l] = synth.softplus(np.random.default_rng(400 + l).standard_normal((Q, g.H)).astype(np.float32))
    cache = fp8_cache(h, g)
    qs = h.Queries(g)
    codes = oracle_codes(g)
    for l in range(2):
        _, out = fp8_layer(h, g, cache, qs, l)
        verify_fp8_full(h, g, l, out, codes=codes, tag=f"fp8-mix-r{r}")

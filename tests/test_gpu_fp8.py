"""GPU parity of the segmented FP8 path against the oracle (needs an MI355X).

The latent rows enter as bf16 values, so the GPU's rotation and quantization
see exactly the oracle's inputs and must reproduce its codes and scales bit
for bit.  The absorbed query is an fp32 MFMA sum on the GPU and an fp64 sum
rounded once to fp32 in the oracle: the two differ in the last bits, so a
code may land one step apart where the rotated value sits on a rounding
boundary (and a scale one binade apart where the segment maximum sits on a
power-of-two boundary); the test bounds those differences instead of
requiring equality.  Scores and top-k sets follow the same rules as the bf16
path (tests/parity.py), each side scoring with its own quantized operands.
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


def test_fp8_absorb_matches_within_one_step():
    h = _gpu()
    for (Q, H, d, r) in ((3, 64, 128, 256), (5, 7, 64, 128), (2, 33, 256, 256)):
        say(f"absorb Q={Q} H={H} d={d} r={r}")
        rng = np.random.default_rng(Q * 100 + H)
        q = synth.round_bf16(rng.standard_normal((Q, H, d)).astype(np.float32))
        W = synth.round_bf16((rng.standard_normal((d, r)) / np.sqrt(r)).astype(np.float32))
        fq = B.absorb_query(h.to_dev(q, torch.bfloat16), h.to_dev(W, torch.bfloat16), fp8=True)
        gc, gs = h.host(fq.codes()), h.host(fq.scales())
        oc, os_ = oracle.absorb_fp8(q, W)
        gv = oracle.e4m3_decode(gc) * np.repeat(gs.astype(np.float64), 128, axis=-1)
        ov = oracle.e4m3_decode(oc) * np.repeat(os_.astype(np.float64), 128, axis=-1)
        # one step of the coarser of the two scales, at the element's binade
        step = np.maximum(np.abs(ov) * 2.0 ** -3, 2.0 ** -9 * np.repeat(np.maximum(gs, os_), 128, axis=-1))
        assert np.all(np.abs(gv - ov) <= step * (1 + 1e-9)), np.max(np.abs(gv - ov) / step)
        same_scale = np.repeat(gs == os_, 128, axis=-1)
        agree = np.mean(gc[same_scale] == oc[same_scale])
        assert np.mean(gs == os_) > 0.95 and agree > 0.99, (np.mean(gs == os_), agree)


def fp8_layer(h, g, cache, qs, l, k=None, k_inner=0):
    fq = B.absorb_query(h.to_dev(g.q[l], torch.bfloat16), h.to_dev(g.W[l], torch.bfloat16), fp8=True)
    out = B.score_topk(cache, qs.seq, qs.pos, qs.max_valid, fq, h.head_weights(g, l), g.k if k is None else k,
                       k_inner=k_inner, keep_scores=True)
    return fq, out


def verify_fp8_full(h, g, l, out, k=None, codes=None, tag=""):
    k = g.k if k is None else k
    codes = oracle_codes(g) if codes is None else codes
    oq, oqs = oracle.absorb_fp8(g.q[l], g.W[l])
    sel, cnt, sc = h.host(out.idx), h.host(out.count), h.host(out.scores)
    for i in range(g.Q):
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
    g = synth.config2()
    cache = fp8_cache(h, g)
    qs = h.Queries(g)
    codes = oracle_codes(g)
    for l in range(g.G):
        _, out = fp8_layer(h, g, cache, qs, l)
        verify_fp8_full(h, g, l, out, codes=codes, tag="fp8-8k")


def test_fp8_ragged_paged_full_and_hs():
    h = _gpu()
    say("fp8 ragged paged: full + HS")
    g = synth.make_decode("f8rag", 61, B=5, lens=(3000, 20000), r=256, H=64, d=128, k=1024, M=4096)
    cache = fp8_cache(h, g)
    qs = h.Queries(g)
    codes = oracle_codes(g)
    _, out = fp8_layer(h, g, cache, qs, 1)
    verify_fp8_full(h, g, 1, out, codes=codes, tag="fp8-rag")
    # HS: the anchor's top-M with its own top-k nested, then every follower
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
                check_topk(a_idx[i], int(a_cnt[i]), oracle.topk(s0, Me), s0, None, Me, rms(s0), f"fp8 anchor q{i}")
                cand = a_idx[i, :Me].astype(np.int64)
                sub = {int(p): s0[p] for p in cand}
                check_topk(a_in[i], int(a_in_cnt[i]), oracle.topk(s0[cand], Ke, pos=cand), sub, cand, Ke, rms(s0),
                           f"fp8 anchor nested q{i}")
            cand = a_idx[i, :Me].astype(np.int32)
            cs_l = oracle.score_fp8(oq[i], oqs[i], g.w[l][i], cc, cs, rows=cand)
            check_scores(fs[i, :Me], cs_l, f"fp8 follower {l} q{i} scores")
            check_topk(fi[i], int(fc[i]), oracle.topk(cs_l, Ke, pos=cand), dict(zip(cand.tolist(), cs_l)), cand, Ke,
                       rms(cs_l), f"fp8 follower {l} q{i} top-k")


def test_fp8_short_empty_and_r128():
    h = _gpu()
    say("fp8 short/empty sequences, r=128, few heads")
    g = synth.make_decode("f8short", 62, B=4, lens=[1, 0, 33, 257], r=128, H=5, d=32, k=16, M=64)
    cache = fp8_cache(h, g)
    qs = h.Queries(g)
    _, out = fp8_layer(h, g, cache, qs, 0)
    verify_fp8_full(h, g, 0, out, tag="fp8-short")

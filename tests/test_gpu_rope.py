"""GPU parity of the RoPE-compatible structured decoder (needs an MI355X).

Rotary sources rotated at append (§A.2), per-frequency complex decoder
coefficients and a dense NoPE decoder absorbed into the post-RoPE query
(§A.2-§A.4), the NoPE output bias added before the ReLU (§A.3).  Rules:
  * append: the oracle rotates in fp64 and the cache holds that value
    rounded once (bf16 straight from fp64, fp32, or fp32 then the FP8
    quantization): bit-exact;
  * bias: products exact in fp64 on both sides, rounded once: bit-exact;
  * absorbed query: bf16 within one bf16 rounding of the oracle's fp64
    value; FP8 codes and scales bit-exact (both sides sum exactly in fp64);
  * scores and top-k: the 1e-2 rule of tests/parity.py against the oracle's
    latent-path score on the same stored operands; on the bf16 path the
    scores also against the oracle's explicit path that rebuilds each
    layer's post-RoPE native key from the unrounded latent (the FP8 path's
    own quantization error is larger than the 1e-2 band, so it is held to
    the oracle's FP8 score only).
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
    print(f"[rope] {msg}", flush=True)
    sys.stdout.flush()


def _gpu():
    import gpu_harness
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    return gpu_harness


def f64_to_bf16(x) -> np.ndarray:
    """Round fp64 values to bf16 in one step (nearest, ties to even)."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8).astype(np.float32)


def rope_cache(h, g, rg, dtype: str):
    """Zeroed pool; every row enters through li_append_latent_rope."""
    dev = h.device()
    r = g.r
    rope = (rg.F, rg.S, rg.base)
    if dtype == "fp8":
        pool = torch.zeros((max(g.num_pages, 1), 64, r), dtype=torch.uint8, device=dev)
        scales = torch.zeros((max(g.num_pages, 1), 64, r // 128), dtype=torch.float32, device=dev)
        cache = B.LatentCache(pool, h.i32(g.block_table), h.i32(g.lens), scales)
        tdt = torch.bfloat16
    else:
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        pool = torch.zeros((max(g.num_pages, 1), 64, r), dtype=tdt, device=dev)
        cache = B.LatentCache(pool, h.i32(g.block_table), h.i32(g.lens))
    for b in range(g.B):
        n = int(g.lens[b])
        if n:
            B.append_latent_rope(cache, h.to_dev(g.latent[b][:n], tdt), h.i32(np.full(n, b)), h.i32(np.arange(n)),
                                 rope)
    return cache


def oracle_rotated(g, rg):
    return [oracle.rope_rotate(g.latent[b][: int(g.lens[b])], np.arange(int(g.lens[b])), rg.F, rg.S, rg.base)
            for b in range(g.B)]


def slot_of(g, b, j):
    return int(g.block_table[b][j // 64]) * 64 + j % 64


def layer_operands(h, g, rg, l, fp8=False):
    """GPU: dense decoder from the structured one, absorbed query, bias."""
    bf = torch.bfloat16
    Wd = B.rope_decoder(h.to_dev(rg.D[l], bf), h.to_dev(rg.Wn[l], bf), (rg.F, rg.S, rg.base))
    q = h.to_dev(g.q[l], bf)
    qt = B.absorb_query(q, Wd, fp8=fp8)
    bias = B.query_bias(q, torch.from_numpy(rg.beta[l]).to(h.device()), rg.d_rope)
    return qt, bias


def test_rope_append_is_bit_exact():
    h = _gpu()
    rg = synth.make_rope(70)
    g = synth.make_decode("rope-app", 70, B=2, lens=[131072, 3000], r=256, H=8, d=128, k=64, M=128, G=1)
    rng = np.random.default_rng(70)
    picks = [np.sort(rng.choice(131072, 3000, replace=False)), np.arange(3000)]
    picks[0][:3] = [0, 1, 131071]
    for dtype in ("bf16", "fp32", "fp8"):
        say(f"append {dtype}")
        dev = h.device()
        if dtype == "fp8":
            pool = torch.zeros((g.num_pages, 64, 256), dtype=torch.uint8, device=dev)
            sc = torch.zeros((g.num_pages, 64, 2), dtype=torch.float32, device=dev)
            cache = B.LatentCache(pool, h.i32(g.block_table), h.i32(g.lens), sc)
        else:
            pool = torch.zeros((g.num_pages, 64, 256), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                               device=dev)
            cache = B.LatentCache(pool, h.i32(g.block_table), h.i32(g.lens))
        tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
        for b in range(2):
            rows = g.latent[b][picks[b]]
            B.append_latent_rope(cache, h.to_dev(rows, tdt), h.i32(np.full(len(rows), b)), h.i32(picks[b]),
                                 (rg.F, rg.S, rg.base))
        got = h.host(cache.pool.float() if dtype == "bf16" else cache.pool).reshape(-1, 256)
        for b in range(2):
            rot = oracle.rope_rotate(g.latent[b][picks[b]], picks[b], rg.F, rg.S, rg.base)
            slots = [slot_of(g, b, int(j)) for j in picks[b]]
            if dtype == "fp8":
                codes, scales = oracle.quantize_rows(rot.astype(np.float32))
                assert np.array_equal(got[slots], codes), f"seq {b}: FP8 codes differ"
                assert np.array_equal(h.host(cache.scales).reshape(-1, 2)[slots], scales), f"seq {b}: scales"
            else:
                want = f64_to_bf16(rot) if dtype == "bf16" else rot.astype(np.float32)
                bad = np.argwhere(got[slots] != want)
                assert bad.size == 0, f"{dtype} seq {b}: {len(bad)} elements differ, first {bad[:3].tolist()}"


def test_rope_decoder_absorption_and_bias():
    h = _gpu()
    for (Q, H, seed) in ((3, 64, 71), (300, 20, 72)):
        say(f"decoder + absorb + bias Q={Q} H={H}")
        rg = synth.make_rope(seed, G=1)
        rng = np.random.default_rng(seed)
        q = synth.round_bf16(rng.standard_normal((Q, H, rg.d)).astype(np.float32))
        g = type("G", (), {"q": [q]})()
        qt, bias = layer_operands(h, g, rg, 0)
        qt_o, b_o = oracle.absorb_rope(q, rg.D[0], rg.Wn[0], rg.beta[0], rg.F, rg.S)
        assert np.array_equal(h.host(bias), b_o.astype(np.float32)), "bias differs"
        gq = h.host(qt.float()).astype(np.float64)
        tol = 2.0 ** -8 * np.abs(qt_o) + 1e-6 * np.max(np.abs(qt_o))
        assert np.all(np.abs(gq - qt_o) <= tol), np.max(np.abs(gq - qt_o) / (np.abs(qt_o) + 1e-30))
        f8, _ = layer_operands(h, g, rg, 0, fp8=True)
        oc, os_ = oracle.quantize_rows(qt_o.astype(np.float32))
        assert np.array_equal(h.host(f8.scales()), os_), "FP8 query scales differ"
        assert np.array_equal(h.host(f8.codes()), oc), "FP8 query codes differ"


def _verify(h, g, rg, l, out, rotated, dtype, queries=None, explicit=False, tag=""):
    qt_o, b_o = oracle.absorb_rope(g.q[l], rg.D[l], rg.Wn[l], rg.beta[l], rg.F, rg.S)
    if dtype == "fp8":
        oq, oqs = oracle.quantize_rows(qt_o.astype(np.float32))
    sel, cnt, sc = h.host(out.idx), h.host(out.count), h.host(out.scores)
    for i in (range(g.Q) if queries is None else queries):
        b = int(g.qseq[i])
        n = oracle.valid_rows(g.qpos[i], g.lens[b])
        if dtype == "fp8":
            cc, cs = rotated[b]
            o = oracle.score_fp8(oq[i], oqs[i], g.w[l][i], cc, cs, n=n, bias=b_o[i])
        else:
            o = oracle.score(qt_o[i], g.w[l][i], rotated[b], n=n, bias=b_o[i])
        check_scores(sc[i, :n], o, f"{tag} layer {l} query {i} scores")
        K = min(g.k, n)
        check_topk(sel[i], int(cnt[i]), oracle.topk(o, K), o, None, K, rms(o), f"{tag} layer {l} query {i} top-k")
        if explicit:
            e = oracle.score_explicit_rope(g.q[l][i], rg.D[l], rg.Wn[l], rg.beta[l], g.w[l][i], g.latent[b][:n],
                                           np.arange(n), rg.F, rg.S, rg.base)
            check_scores(sc[i, :n], e, f"{tag} layer {l} query {i} vs rebuilt post-RoPE keys")


def _stored(g, rg, dtype):
    rot = oracle_rotated(g, rg)
    if dtype == "fp8":
        return [oracle.quantize_rows(x.astype(np.float32)) for x in rot]
    return [f64_to_bf16(x) for x in rot]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_rope_decode_full_and_hs(dtype):
    h = _gpu()
    rg = synth.make_rope(73)
    g = synth.make_decode(f"rope-dec-{dtype}", 73, B=3, lens=[2000, 9000, 17000], r=256, H=64, d=128, k=1024,
                          M=4096)
    say(f"decode {dtype}: cache")
    cache = rope_cache(h, g, rg, dtype)
    qs = h.Queries(g)
    stored = _stored(g, rg, dtype)
    ops = [layer_operands(h, g, rg, l, fp8=(dtype == "fp8")) for l in range(g.G)]
    for l in (0, 1):
        say(f"decode {dtype}: full layer {l}")
        qt, bias = ops[l]
        out = B.score_topk(cache, qs.seq, qs.pos, qs.max_valid, qt, h.head_weights(g, l), g.k, keep_scores=True,
                           bias=bias)
        _verify(h, g, rg, l, out, stored, dtype, explicit=(l == 0 and dtype == "bf16"), tag=f"rope-{dtype}")
    say(f"decode {dtype}: HS")
    qt0, b0 = ops[0]
    anchor = B.score_topk(cache, qs.seq, qs.pos, qs.max_valid, qt0, h.head_weights(g, 0), g.M, k_inner=g.k,
                          keep_scores=True, bias=b0)
    a_idx, a_cnt = h.host(anchor.idx), h.host(anchor.count)
    for l in range(1, g.G):
        qt, bias = ops[l]
        fo = B.hs_select(cache, qs.seq, qs.pos, qs.max_valid, anchor.idx, anchor.count, qt, h.head_weights(g, l), g.k,
                         keep_scores=True, bias=bias)
        qt_o, b_o = oracle.absorb_rope(g.q[l], rg.D[l], rg.Wn[l], rg.beta[l], rg.F, rg.S)
        if dtype == "fp8":
            oq, oqs = oracle.quantize_rows(qt_o.astype(np.float32))
        fi, fc, fs = h.host(fo.idx), h.host(fo.count), h.host(fo.scores)
        for i in range(g.Q):
            b = int(g.qseq[i])
            n = oracle.valid_rows(g.qpos[i], g.lens[b])
            Me, Ke = min(g.M, n), min(g.k, min(g.M, n))
            assert int(a_cnt[i]) == Me
            cand = a_idx[i, :Me].astype(np.int32)
            if dtype == "fp8":
                cc, cs = stored[b]
                o = oracle.score_fp8(oq[i], oqs[i], g.w[l][i], cc, cs, rows=cand, bias=b_o[i])
            else:
                o = oracle.score(qt_o[i], g.w[l][i], stored[b], rows=cand, bias=b_o[i])
            check_scores(fs[i, :Me], o, f"rope-{dtype} follower {l} q{i} scores")
            check_topk(fi[i], int(fc[i]), oracle.topk(o, Ke, pos=cand), dict(zip(cand.tolist(), o)), cand, Ke,
                       rms(o), f"rope-{dtype} follower {l} q{i} top-k")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_rope_decode_long_context_b4_n131072(dtype):
    """The long-context shape (4 sequences of 131072 rows) through the
    structured decoder, in the launch configuration the benchmark times: a
    rotated cache, one layer's absorbed query with its bias, every score and
    the selection."""
    h = _gpu()
    rg = synth.make_rope(74)
    g = synth.make_decode(f"rope-long-{dtype}", 74, B=4, lens=[131072] * 4, r=256, H=64, d=128, k=2048, M=8192)
    say(f"long context {dtype}: cache")
    cache = rope_cache(h, g, rg, dtype)
    qs = h.Queries(g)
    stored = _stored(g, rg, dtype)
    qt, bias = layer_operands(h, g, rg, 2, fp8=(dtype == "fp8"))
    say(f"long context {dtype}: full layer 2")
    out = B.score_topk(cache, qs.seq, qs.pos, qs.max_valid, qt, h.head_weights(g, 2), g.k, keep_scores=True,
                       bias=bias)
    _verify(h, g, rg, 2, out, stored, dtype, tag=f"rope-long-{dtype}")
    del cache
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_rope_prefill_sampled(dtype):
    """The chunked-prefill workload (4096 queries at the end of a 65536-row
    cache, 4 layers) through the structured decoder: 64 evenly spaced query
    rows of every layer against the oracle; on the bf16 path the first and
    last sampled rows of layer 0 also against rebuilt post-RoPE keys."""
    h = _gpu()
    rg = synth.make_rope(74)
    g = synth.make_prefill(f"rope-pf-{dtype}", 74, N=65536, Qn=4096, r=256, H=64, d=128, G=4, k=2048)
    say(f"prefill {dtype}: cache")
    cache = rope_cache(h, g, rg, dtype)
    qs = h.Queries(g)
    stored = _stored(g, rg, dtype)
    sample = h.prefill_sample(g.Q)
    assert len(sample) == 64 and sample[0] == 0 and sample[-1] == g.Q - 1
    for l in range(g.G):
        say(f"prefill {dtype}: layer {l}")
        qt, bias = layer_operands(h, g, rg, l, fp8=(dtype == "fp8"))
        out = B.score_topk(cache, qs.seq, qs.pos, qs.max_valid, qt, h.head_weights(g, l), g.k, keep_scores=True,
                           bias=bias)
        _verify(h, g, rg, l, out, stored, dtype, queries=sample, tag=f"rope-pf-{dtype}")
        if dtype == "bf16" and l == 0:
            _verify(h, g, rg, l, out, stored, dtype, queries=[sample[0], sample[-1]], explicit=True,
                    tag=f"rope-pf-{dtype}")
        del out
        torch.cuda.empty_cache()


def test_bias_on_the_register_staged_and_fp32_paths():
    """r = 128 contiguous decode (register-staged kernel) and the fp32 cache
    path, each with a bias of both signs (the ReLU cuts some heads)."""
    h = _gpu()
    for (r, dt) in ((128, "bf16"), (64, "fp32")):
        say(f"bias r={r} {dt}")
        g = synth.make_decode(f"bias-{r}", 75 + r, B=2, lens=[5000, 700], r=r, H=48, d=r, k=256, M=512, G=1,
                              dtype=dt)
        cache = h.build_cache(g)
        qs = h.Queries(g)
        rng = np.random.default_rng(r)
        bias_np = (rng.standard_normal((g.Q, g.H)) * 4.0).astype(np.float32)
        qt = h.absorbed(g, 0)
        out = B.score_topk(cache, qs.seq, qs.pos, qs.max_valid, qt, h.head_weights(g, 0), g.k, keep_scores=True,
                           bias=torch.from_numpy(bias_np).to(h.device()))
        qt_o = oracle.absorb(g.q[0], g.W[0])
        sel, cnt, sc = h.host(out.idx), h.host(out.count), h.host(out.scores)
        for i in range(g.Q):
            b = int(g.qseq[i])
            n = oracle.valid_rows(g.qpos[i], g.lens[b])
            o = oracle.score(qt_o[i], g.w[0][i], g.latent[b], n=n, bias=bias_np[i])
            check_scores(sc[i, :n], o, f"bias r={r} q{i} scores")
            K = min(g.k, n)
            check_topk(sel[i], int(cnt[i]), oracle.topk(o, K), o, None, K, rms(o), f"bias r={r} q{i} top-k")


@pytest.mark.parametrize("H", [1, 64])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("many", [False, True])
def test_bias_enters_exactly(H, dtype, many):
    """On all-zero latent rows every score is sum_h w_h max(b_h, 0): the bias
    must reach the ReLU as the exact fp32 value (the prefill kernels build it
    from three bf16 parts inside the MFMA).  One head: the score is one fp32
    product, within 2^-22; 64 heads: within the fp32 sum's rounding (1e-5 of
    the sum of magnitudes), which also catches a head mapped to another's
    bias.  Biases span 2^-12..2^12, weights take both signs."""
    h = _gpu()
    dev = h.device()
    say(f"bias exact H={H} {dtype} {'prefill' if many else 'decode'}")
    rng = np.random.default_rng(9100 + H + (7 if many else 0) + (3 if dtype == "fp8" else 0))
    r, d = 256, 128
    lens = [300, 170]
    pages = [(n + 63) // 64 for n in lens]
    bt = np.full((len(lens), max(pages)), -1, dtype=np.int32)
    nxt = 0
    for b, p in enumerate(pages):
        bt[b, :p] = np.arange(nxt, nxt + p)
        nxt += p
    if many:  # 8 queries per sequence at spread positions: the prefill kernels
        qseq = np.repeat(np.arange(len(lens)), 8)
        qpos = np.concatenate([np.linspace(0, n - 1, 8).astype(np.int64) for n in lens])
    else:
        qseq = np.arange(len(lens))
        qpos = np.asarray(lens) - 1
    Q = len(qseq)
    if dtype == "fp8":
        cache = B.LatentCache(torch.zeros((nxt, 64, r), dtype=torch.uint8, device=dev), h.i32(bt), h.i32(lens),
                              torch.zeros((nxt, 64, r // 128), dtype=torch.float32, device=dev))
        q = h.to_dev(rng.standard_normal((Q, H, d)).astype(np.float32), torch.bfloat16)
        W = h.to_dev((rng.standard_normal((d, r)) / 16).astype(np.float32), torch.bfloat16)
        qt = B.absorb_query(q, W, fp8=True)
    else:
        cache = B.LatentCache(torch.zeros((nxt, 64, r), dtype=torch.bfloat16, device=dev), h.i32(bt), h.i32(lens))
        qt = h.to_dev(rng.standard_normal((Q, H, r)).astype(np.float32), torch.bfloat16)
    w = rng.standard_normal((Q, H)).astype(np.float32)
    bias = (rng.standard_normal((Q, H)) * np.exp2(rng.uniform(-12, 12, (Q, H)))).astype(np.float32)
    nvalid = np.minimum(qpos + 1, np.asarray(lens)[qseq])
    maxv = int(nvalid.max())
    out = B.score_topk(cache, h.i32(qseq), h.i32(qpos), maxv, qt, torch.from_numpy(w).to(dev), 64,
                       keep_scores=True, bias=torch.from_numpy(bias).to(dev))
    got = out.scores.cpu().numpy()
    terms = w.astype(np.float64) * np.maximum(bias.astype(np.float64), 0.0)
    want = terms.sum(axis=1)
    mag = np.abs(terms).sum(axis=1)
    tol = mag * (2.0 ** -22 if H == 1 else 1e-5) + 1e-30
    for i in range(Q):
        row = got[i, : nvalid[i]].astype(np.float64)
        err = np.abs(row - want[i]).max()
        assert err <= tol[i], f"query {i}: max error {err:.3e} > {tol[i]:.3e} (score {want[i]:.6e})"

"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every case uses seeded synthetic inputs; the oracle sees fp64 copies of the
exact bits the GPU sees.  Comparison rules are in parity.py (scores within
1e-2 relative with an RMS floor; top-k sets exact up to swaps inside one
tolerance band of the cut-off).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from parity import STRICT_FLOOR, check_scores, check_topk, overlap, rms
from sparse_attention_token_absorb_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(msg: str) -> None:
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from sparse_attention_token_absorb_amd import binding
    binding.lib()  # must load: there is no other path
    yield


def H():
    import gpu_harness
    return gpu_harness


# ----------------------------------------------------------------------------
# Verification helpers
# ----------------------------------------------------------------------------
def _floor(g, l):
    """Score-rule floor: strict when the layer has many heads and no negative
    head weight, so that a score is a sum of many non-negative terms and its
    rounding error stays relative to it.  With few heads a small score can be
    one head whose dot product sits just above the ReLU cut, and the one
    bf16 rounding of the absorbed query is then large against it."""
    return STRICT_FLOOR if g.H >= 32 and np.all(np.asarray(g.w[l]) >= 0) else 1.0


def verify_full(g, l, res, k=None, queries=None, tag=""):
    h = H()
    k = g.k if k is None else k
    sel, cnt = h.host(res.idx), h.host(res.count)
    sc = h.host(res.scores) if res.scores is not None else None
    qi = list(range(g.Q)) if queries is None else list(queries)
    orc = oracle.full_layer(g.q[l], g.W[l], g.w[l], g.latent, g.qseq, g.qpos, g.lens, k, qi)
    swaps = 0
    worst = 0.0
    for i, o in zip(qi, orc):
        n = len(o.scores)
        if sc is not None:
            worst = max(worst, check_scores(sc[i, :n], o.scores, f"{tag} layer {l} query {i} scores", _floor(g, l)))
        swaps += check_topk(sel[i], int(cnt[i]), o.sel, o.scores, None, min(k, n), rms(o.scores),
                            f"{tag} layer {l} query {i} top-{k}")
    if sc is not None:
        say(f"{tag} layer {l}: worst relative score error {worst:.2e} (rows above 1e-3 RMS), {swaps} band swaps")
    return swaps, orc


def verify_hs(g, anchor, followers, M=None, k=None, tag=""):
    h = H()
    M = g.M if M is None else M
    k = g.k if k is None else k
    a_idx, a_cnt = h.host(anchor.idx), h.host(anchor.count)
    a_in, a_in_cnt = h.host(anchor.idx_inner), h.host(anchor.count_inner)
    f_out = [(h.host(f.idx), h.host(f.count), h.host(f.scores) if f.scores is not None else None) for f in followers]
    for i in range(g.Q):
        b = int(g.qseq[i])
        n = oracle.valid_rows(g.qpos[i], g.lens[b])
        s0 = oracle.score(oracle.absorb(g.q[0][i], g.W[0]), g.w[0][i], g.latent[b], n)
        rho0 = rms(s0)
        Me = min(M, n)
        check_topk(a_idx[i], int(a_cnt[i]), oracle.topk(s0, Me), s0, None, Me, rho0, f"{tag} anchor top-M q{i}")
        cand = a_idx[i, :Me].astype(np.int64)
        Ke = min(k, Me)
        sub = {int(p): s0[p] for p in cand}
        check_topk(a_in[i], int(a_in_cnt[i]), oracle.topk(s0[cand], Ke, pos=cand), sub, cand, Ke, rho0,
                   f"{tag} anchor nested top-k q{i}")
        for l, (fi, fc, fs) in enumerate(f_out, start=1):
            cs = oracle.score(oracle.absorb(g.q[l][i], g.W[l]), g.w[l][i], g.latent[b], rows=cand)
            if fs is not None:
                check_scores(fs[i, :Me], cs, f"{tag} follower {l} q{i} candidate scores", _floor(g, l))
            check_topk(fi[i], int(fc[i]), oracle.topk(cs, Ke, pos=cand), dict(zip(cand.tolist(), cs)), cand, Ke,
                       rms(cs), f"{tag} follower {l} q{i} top-k")


# ----------------------------------------------------------------------------
# Boundary pieces
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,r", [("bf16", 256), ("bf16", 64), ("fp32", 64), ("fp32", 20)])
def test_append_latent_bit_exact(dtype, r):
    h = H()
    say(f"append {dtype} r={r}")
    g = synth.make_decode("append", 31, B=3, lens=[130, 64, 1], r=r, H=4, d=32, k=8, M=16, dtype=dtype,
                          n_heavy=1, paged=True)
    cache = h.build_cache(g, rows_per_append=50)
    torch.cuda.synchronize()
    pool = cache.pool.float().cpu().numpy() if dtype == "bf16" else cache.pool.cpu().numpy()
    used = set()
    for b in range(g.B):
        for j in range(int(g.lens[b])):
            page = int(g.block_table[b, j // 64])
            used.add((page, j % 64))
            assert np.array_equal(pool[page, j % 64].view(np.uint32), g.latent[b][j].view(np.uint32)), (b, j)
    for p in range(g.num_pages):
        for s in range(64):
            if (p, s) not in used:
                assert not pool[p, s].any(), "append wrote outside its slots"


@pytest.mark.parametrize("dtype,d,r,Q,Hh", [("bf16", 128, 256, 3, 64), ("bf16", 32, 64, 5, 4), ("bf16", 64, 128, 2, 48),
                                            ("bf16", 256, 256, 1, 7), ("fp32", 32, 64, 2, 4), ("fp32", 13, 9, 3, 3)])
def test_absorb_parity(dtype, d, r, Q, Hh):
    h = H()
    say(f"absorb {dtype} d={d} r={r} Q={Q} H={Hh}")
    rng = np.random.default_rng(d * 1000 + r)
    q = rng.standard_normal((Q, Hh, d)).astype(np.float32)
    W = (rng.standard_normal((d, r)) / np.sqrt(r)).astype(np.float32)
    if dtype == "bf16":
        q, W = synth.round_bf16(q), synth.round_bf16(W)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    from sparse_attention_token_absorb_amd import binding as B
    got = h.host(B.absorb_query(h.to_dev(q, tdt), h.to_dev(W, tdt)).float())
    ref = oracle.absorb(q, W)
    mag = np.abs(q.astype(np.float64)) @ np.abs(W.astype(np.float64))
    # one bf16 rounding (half an ulp, <= 2^-8 relative) on top of fp32 accumulation
    tol = (2.0 ** -8) * np.abs(ref) + 1e-6 * mag if dtype == "bf16" else 1e-6 * mag + 1e-30
    assert np.all(np.abs(got - ref) <= tol), float(np.max(np.abs(got - ref) - tol))


# ----------------------------------------------------------------------------
# The five workloads
# ----------------------------------------------------------------------------
def test_tiny_fp32_n512_full_and_hs():
    h = H()
    g = synth.tiny_fp32_n512()
    say("tiny fp32 N=512: cache")
    cache = h.build_cache(g)
    qs = h.Queries(g)
    for l in range(g.G):
        say(f"tiny fp32 full layer {l}")
        res = h.full_layer(g, cache, qs, l)
        verify_full(g, l, res, tag="tiny fp32")
    say("tiny fp32 HS")
    anchor, followers = h.hs_group(g, cache, qs)
    verify_hs(g, anchor, followers, tag="tiny fp32")


def test_tiny_n512_through_the_bf16_kernels():
    """The tiny configuration's cache is fp32 and runs on the fp32 kernel;
    its inputs rounded once to bf16 also run through the bf16 MFMA kernels
    (the register-staged one scores its contiguous r = 64 prefix, the LDS
    ring the HS followers' gathered rows), against the oracle on the same
    rounded values."""
    import dataclasses
    h = H()
    g0 = synth.tiny_fp32_n512()
    rb = synth.round_bf16
    g = dataclasses.replace(g0, name=g0.name + "-bf16", dtype="bf16", latent=[rb(x) for x in g0.latent],
                            q=[rb(x) for x in g0.q], W=[rb(x) for x in g0.W])
    say("tiny N=512 on bf16 copies: cache")
    cache = h.build_cache(g)
    qs = h.Queries(g)
    for l in range(g.G):
        say(f"tiny bf16 full layer {l}")
        verify_full(g, l, h.full_layer(g, cache, qs, l), tag="tiny bf16")
    say("tiny bf16 HS")
    anchor, followers = h.hs_group(g, cache, qs)
    verify_hs(g, anchor, followers, tag="tiny bf16")


def test_decode_b1_n8192_bf16():
    h = H()
    g = synth.decode_b1_n8192()
    say("decode B=1 N=8192 bf16: cache")
    cache = h.build_cache(g)
    qs = h.Queries(g)
    full = []
    for l in range(g.G):
        say(f"decode 8K full layer {l}")
        res = h.full_layer(g, cache, qs, l)
        verify_full(g, l, res, tag="decode 8K")
        full.append(h.host(res.idx))
    # M = n: HS is full LatentIndex (up to exact-tie / tolerance swaps)
    say("decode 8K HS with M = N")
    anchor, followers = h.hs_group(g, cache, qs, M=8192)
    verify_hs(g, anchor, followers, M=8192, tag="decode 8K M=N")


def test_ragged_paged_b16_hs_and_full():
    h = H()
    g = synth.ragged_paged_b16()
    say(f"ragged paged B={g.B} lens {int(g.lens.min())}..{int(g.lens.max())}: cache")
    cache = h.build_cache(g)
    qs = h.Queries(g)
    say("ragged paged HS")
    anchor, followers = h.hs_group(g, cache, qs)
    verify_hs(g, anchor, followers, tag="ragged paged")
    ov = []
    for l in range(g.G):
        say(f"ragged paged full layer {l}")
        res = h.full_layer(g, cache, qs, l)
        verify_full(g, l, res, tag="ragged paged")
        hs_sel = h.host(anchor.idx_inner) if l == 0 else h.host(followers[l - 1].idx)
        full_sel = h.host(res.idx)
        ov += [overlap(hs_sel[i][hs_sel[i] >= 0], full_sel[i][full_sel[i] >= 0]) for i in range(g.Q)]
    say(f"ragged paged HS-vs-full top-k overlap mean {np.mean(ov):.4f} (reported, not pinned)")


def test_long_context_b4_n131072_all_three_ways():
    """(b) full LatentIndex, (c) HS and (a) the per-layer baseline on keys that
    are each layer's decoder applied to the same latent (rounded once to
    bf16).  Absorption is exact for those effective keys (summary page,
    §3.1), so (a)'s selection must agree with (b)'s oracle selection up to
    swaps inside the tolerance band."""
    h = H()
    g = synth.long_context_b4()
    say("long context B=4 N=131072: cache")
    cache = h.build_cache(g)
    qs = h.Queries(g)
    orc_b = []
    for l in range(g.G):
        say(f"long context (b) full layer {l}")
        _, orc = verify_full(g, l, h.full_layer(g, cache, qs, l), tag="long context (b)")
        orc_b.append(orc)
    say("long context (c) HS M=8192")
    anchor, followers = h.hs_group(g, cache, qs)
    verify_hs(g, anchor, followers, tag="long context (c)")
    del cache
    torch.cuda.empty_cache()
    from sparse_attention_token_absorb_amd import binding as B
    for l in range(g.G):
        say(f"long context (a) per-layer key cache layer {l}")
        kc = h.build_cache(g, latent=g.keys_a[l], r=g.d)
        q = h.to_dev(g.q[l], torch.bfloat16)
        res = B.score_topk(kc, qs.seq, qs.pos, qs.max_valid, q, h.head_weights(g, l), g.k, keep_scores=True)
        sel, cnt, sc = h.host(res.idx), h.host(res.count), h.host(res.scores)
        orc_a = oracle.baseline_layer(g.q[l], g.w[l], g.keys_a[l], g.qseq, g.qpos, g.lens, g.k)
        for i in range(g.Q):
            s = orc_a[i].scores
            check_scores(sc[i, :len(s)], s, f"long context (a) layer {l} q{i}")
            check_topk(sel[i], int(cnt[i]), orc_a[i].sel, s, None, g.k, rms(s), f"long context (a) layer {l} q{i}")
            # the baseline and the latent path select the same rows up to the band
            ob = orc_b[l][i]
            swaps = check_topk(sel[i], int(cnt[i]), ob.sel, ob.scores, None, g.k, rms(ob.scores),
                               f"long context (a) vs (b) layer {l} q{i}")
            say(f"(a) vs (b) layer {l} q{i}: {swaps} band swaps of {g.k}")
        del kc


@pytest.mark.parametrize("seed", [40, 400])
def test_long_context_b4_n131072_other_requests(seed):
    """The timing protocol of the LatentIndex summary page (§C.4) runs three
    requests per method and length; the long-context workload's other two
    seeded requests: one full LatentIndex layer (every score) and the HS
    group (anchor top-8192 with its nested top-2048, 3 followers)."""
    h = H()
    g = synth.long_context_b4(seed=seed, keys_a=False)
    say(f"long context seed {seed}: cache")
    cache = h.build_cache(g)
    qs = h.Queries(g)
    verify_full(g, 1, h.full_layer(g, cache, qs, 1), tag=f"long context seed {seed} (b)")
    say(f"long context seed {seed}: HS M=8192")
    anchor, followers = h.hs_group(g, cache, qs)
    verify_hs(g, anchor, followers, tag=f"long context seed {seed} (c)")
    del cache
    torch.cuda.empty_cache()


@pytest.mark.parametrize("N", [12288, 16384])
def test_decode_b4_sweep_contexts_up_to_16384(N):
    """The benchmark's context sweep (8K-128K) at the lengths where a few
    queries' rows of 8193..16384 scores are selected by one workgroup per
    query that counts the keys itself: every layer of the group full (every
    score), then the HS group (anchor top-8192 with its nested top-2048)."""
    h = H()
    g = synth.long_context_b4(seed=16, N=N, keys_a=False)
    say(f"sweep context N={N}: cache")
    cache = h.build_cache(g)
    qs = h.Queries(g)
    for l in range(g.G):
        verify_full(g, l, h.full_layer(g, cache, qs, l), tag=f"sweep N={N} layer {l}")
    anchor, followers = h.hs_group(g, cache, qs)
    verify_hs(g, anchor, followers, tag=f"sweep N={N} HS")
    del cache
    torch.cuda.empty_cache()


def test_chunked_prefill_q4096_sampled_rows():
    h = H()
    g = synth.chunked_prefill_q4096()
    say("chunked prefill Q=4096 N=65536: cache")
    cache = h.build_cache(g)
    qs = h.Queries(g)
    sample = h.prefill_sample(g.Q)
    assert len(sample) == 64 and sample[0] == 0 and sample[-1] == g.Q - 1
    for l in range(g.G):
        say(f"chunked prefill layer {l}")
        res = h.full_layer(g, cache, qs, l)
        verify_full(g, l, res, queries=sample, tag="chunked prefill")
        cnt = h.host(res.count)
        exp = np.minimum(g.k, np.minimum(g.qpos + 1, g.lens[0]))
        assert np.array_equal(cnt, exp)
        del res
        torch.cuda.empty_cache()


# ----------------------------------------------------------------------------
# Edge cases
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("r,Hh", [(64, 4), (128, 32), (256, 48), (256, 64), (128, 64)])
def test_widths_and_heads(r, Hh):
    h = H()
    say(f"widths r={r} H={Hh}")
    g = synth.make_decode(f"w{r}h{Hh}", 40 + r + Hh, B=2, lens=[3000, 777], r=r, H=Hh, d=128, k=300, M=1000)
    cache = h.build_cache(g)
    qs = h.Queries(g)
    for l in (0, 3):
        verify_full(g, l, h.full_layer(g, cache, qs, l), tag=f"r{r}H{Hh}")
    anchor, followers = h.hs_group(g, cache, qs)
    verify_hs(g, anchor, followers, tag=f"r{r}H{Hh}")


def test_short_and_empty_sequences():
    h = H()
    say("short/empty sequences")
    g = synth.make_decode("short", 50, B=4, lens=[100, 1, 65, 0], r=256, H=64, d=128, k=256, M=512)
    g.qpos = np.maximum(g.qpos, 0).astype(np.int32)
    cache = h.build_cache(g)
    qs = h.Queries(g)
    res = h.full_layer(g, cache, qs, 1)
    cnt = h.host(res.count)
    assert cnt.tolist() == [100, 1, 65, 0]
    assert np.all(h.host(res.idx)[3] == -1)
    verify_full(g, 1, res, queries=[0, 1, 2], tag="short")
    anchor, followers = h.hs_group(g, cache, qs)
    assert h.host(anchor.count).tolist() == [100, 1, 65, 0]
    for f in followers:
        assert h.host(f.count).tolist() == [100, 1, 65, 0]
    verify_hs(g, anchor, followers, tag="short")


def test_mid_prefix_positions():
    """Queries in the middle of their sequences only see their causal prefix."""
    h = H()
    say("mid-prefix positions")
    g = synth.make_decode("mid", 51, B=2, lens=[5000, 4000], r=128, H=16, d=64, k=512, M=2048)
    g.qpos = np.array([2999, 100], dtype=np.int32)
    cache = h.build_cache(g)
    qs = h.Queries(g)
    res = h.full_layer(g, cache, qs, 2)
    assert h.host(res.count).tolist() == [512, 101]
    verify_full(g, 2, res, tag="mid")


def test_exact_ties_zero_rows_negative_weights():
    h = H()
    say("ties / zero rows / negative weights")
    g = synth.make_decode("ties", 52, B=2, lens=[20000, 3000], r=256, H=64, d=128, k=2048, M=4096)
    rng = np.random.default_rng(5)
    lat0 = g.latent[0]
    lat0[rng.choice(20000, 6000, replace=False)] = 0.0            # all-zero rows: score exactly 0
    dup = rng.choice(20000, 300, replace=False)
    lat0[dup] = lat0[dup[0]]                                       # 300 copies of one row
    g.latent[1][:] = g.latent[1][0]                                # every row identical
    g.w[2][:, ::3] *= -1.0                                         # mixed-sign head weights
    cache = h.build_cache(g)
    qs = h.Queries(g)
    for l in range(g.G):
        verify_full(g, l, h.full_layer(g, cache, qs, l), tag="ties")
    anchor, followers = h.hs_group(g, cache, qs)
    verify_hs(g, anchor, followers, tag="ties")


def test_many_queries_mixed_sequences_and_overflow():
    """Prefill kernel with workgroups whose queries sit in different sequences,
    and a threshold bin far larger than the candidate buffer."""
    h = H()
    say("mixed-sequence prefill workgroups + candidate overflow")
    g = synth.make_decode("mixed", 53, B=3, lens=[20000, 9000, 17000], r=256, H=64, d=128, k=2048, M=4096)
    Q = 72
    g.qseq = np.array([i % 3 for i in range(Q)], dtype=np.int32)
    rng = np.random.default_rng(9)
    g.qpos = np.array([rng.integers(0, int(g.lens[b])) for b in g.qseq], dtype=np.int32)
    g.qpos[:3] = g.lens - 1
    g.latent[0][:19000] = 0.0  # most scores exactly zero in sequence 0
    for l in range(g.G):
        g.q[l] = synth.round_bf16(np.random.default_rng(100 + l).standard_normal((Q, g.H, g.d)).astype(np.float32))
        g.w[l] = synth.softplus(np.random.default_rng(200 + l).standard_normal((Q, g.H)).astype(np.float32))
    cache = h.build_cache(g)
    qs = h.Queries(g)
    for l in (0, 1):
        verify_full(g, l, h.full_layer(g, cache, qs, l), tag="mixed")


def test_hs_budget_equal_k_is_index_reuse():
    """M = k: every follower returns exactly the anchor's candidate set."""
    h = H()
    say("HS M = k")
    g = synth.make_decode("reuse", 54, B=2, lens=[10000, 6000], r=256, H=64, d=128, k=1024, M=1024)
    cache = h.build_cache(g)
    qs = h.Queries(g)
    anchor, followers = h.hs_group(g, cache, qs, M=1024, k=1024)
    a = h.host(anchor.idx)
    for f in followers:
        fi = h.host(f.idx)
        for i in range(g.Q):
            assert set(fi[i].tolist()) == set(a[i].tolist())
    verify_hs(g, anchor, followers, M=1024, k=1024, tag="reuse")


def test_repeat_calls_are_deterministic_in_sets():
    """Two identical calls give identical scores and equally valid sets."""
    h = H()
    say("repeat calls")
    g = synth.make_decode("rep", 55, B=1, lens=[50000], r=256, H=64, d=128, k=2048, M=8192)
    cache = h.build_cache(g)
    qs = h.Queries(g)
    r1 = h.full_layer(g, cache, qs, 0)
    r2 = h.full_layer(g, cache, qs, 0)
    assert np.array_equal(h.host(r1.scores), h.host(r2.scores))
    assert set(h.host(r1.idx)[0].tolist()) == set(h.host(r2.idx)[0].tolist())


def test_long_rows_with_massive_ties():
    """Few queries, long rows, and a threshold digit shared by ~40K rows:
    the tie list overflows LDS and the final pass re-reads the row."""
    h = H()
    say("long rows + massive ties")
    g = synth.make_decode("bigties", 56, B=2, lens=[40000, 30000], r=128, H=16, d=64, k=2048, M=8192)
    g.latent[0][:39000] = 0.0
    g.latent[1][:] = g.latent[1][7]
    cache = h.build_cache(g)
    qs = h.Queries(g)
    for l in (0, 1):
        verify_full(g, l, h.full_layer(g, cache, qs, l), tag="bigties")
    anchor, followers = h.hs_group(g, cache, qs)
    verify_hs(g, anchor, followers, tag="bigties")


def test_hs_nested_selection_on_a_shared_tie_digit():
    """The anchor's top-k and top-M thresholds fall on the same run of equal
    scores (6000 identical rows), short enough to be resolved in LDS: the
    nested set must still lie inside the outer one."""
    h = H()
    say("HS nested selection, shared tie digit")
    g = synth.make_decode("nested", 57, B=1, lens=[20000], r=256, H=64, d=128, k=2048, M=4096)
    lat = g.latent[0]
    lat[7500:] = 0.0
    s = oracle.score(oracle.absorb(g.q[0][0], g.W[0]), g.w[0][0], lat, 20000)
    order = np.argsort(-s[:7500], kind="stable")
    lat[order[1500:7500]] = lat[order[1500]]
    cache = h.build_cache(g)
    qs = h.Queries(g)
    anchor, followers = h.hs_group(g, cache, qs, M=4096, k=2048)
    outer = set(h.host(anchor.idx)[0, :4096].tolist())
    inner = set(h.host(anchor.idx_inner)[0, :2048].tolist())
    assert int(h.host(anchor.count)[0]) == 4096 and int(h.host(anchor.count_inner)[0]) == 2048
    assert len(inner) == 2048 and inner <= outer
    verify_hs(g, anchor, followers, M=4096, k=2048, tag="nested")


def test_hs_anchor_tie_digit_wider_than_lds():
    """Plain normal rows give a narrow score distribution: more rows share the
    anchor's top-M threshold digit than the LDS tie list holds, but all of
    them fit the workspace's candidate list, which is ranked instead of the
    whole row."""
    h = H()
    say("HS anchor, tie digit wider than LDS")
    g = synth.make_decode("widetie", 59, B=1, lens=[131072], r=256, H=64, d=128, k=2048, M=8192, G=2,
                          heavy_frac=0.0, structure=False)
    s = oracle.score(oracle.absorb(g.q[0][0], g.W[0]), g.w[0][0], g.latent[0], 131072)
    key = np.sort(s)[-8192].astype(np.float32).view(np.uint32) >> 20
    ties = int(np.sum((s.astype(np.float32).view(np.uint32) >> 20) == key))
    assert ties > 8192, ties  # the case this test is for
    cache = h.build_cache(g)
    qs = h.Queries(g)
    anchor, followers = h.hs_group(g, cache, qs)
    verify_hs(g, anchor, followers, tag="widetie")


def test_largest_budgets():
    """k = 65536 (the largest budget the selectors take) over sequences longer
    and shorter than it, and HS with M = 65536, k = 32768."""
    h = H()
    say("largest budgets")
    g = synth.make_decode("maxk", 60, B=2, lens=[70000, 40000], r=256, H=64, d=128, k=65536, M=65536, G=2)
    cache = h.build_cache(g)
    qs = h.Queries(g)
    res = h.full_layer(g, cache, qs, 0)
    verify_full(g, 0, res, tag="maxk")
    assert np.array_equal(h.host(res.count), np.minimum(65536, g.lens))
    anchor, followers = h.hs_group(g, cache, qs, M=65536, k=32768)
    verify_hs(g, anchor, followers, M=65536, k=32768, tag="maxk-hs")


def test_many_queries_rows_between_8k_and_16k():
    """Prefill-style selection whose rows fit the LDS key cache (8K < n <= 16K),
    with a run of equal scores at the threshold."""
    h = H()
    say("many queries, 8K-16K rows")
    g = synth.make_decode("mid", 58, B=2, lens=[12000, 9000], r=256, H=64, d=128, k=2048, M=4096)
    Q = 40
    g.qseq = np.array([i % 2 for i in range(Q)], dtype=np.int32)
    rng = np.random.default_rng(11)
    g.qpos = np.array([rng.integers(8500, int(g.lens[b])) for b in g.qseq], dtype=np.int32)
    g.qpos[:2] = g.lens - 1
    g.latent[1][:5000] = g.latent[1][5000]  # 5001 identical rows in sequence 1
    for l in range(g.G):
        g.q[l] = synth.round_bf16(np.random.default_rng(300 + l).standard_normal((Q, g.H, g.d)).astype(np.float32))
        g.w[l] = synth.softplus(np.random.default_rng(400 + l).standard_normal((Q, g.H)).astype(np.float32))
    cache = h.build_cache(g)
    qs = h.Queries(g)
    for l in (0, 1):
        verify_full(g, l, h.full_layer(g, cache, qs, l), tag="mid")

"""GPU: device-resident indices outside the cache are bounded by the kernels.

Sequence ids, positions and page ids live in device memory, where the host
cannot check them.  An append whose row maps outside the cache writes
nothing; scoring clamps sequence and page ids into range, so a query with
garbage indices gets meaningless scores but the call completes and every
other query of the call is unaffected.
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
    print(f"[bounds] {msg}", flush=True)
    sys.stdout.flush()


def _gpu():
    import gpu_harness
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    return gpu_harness


@pytest.mark.parametrize("kind", ["bf16", "fp32", "fp8", "rope"])
def test_append_skips_rows_outside_the_cache(kind):
    h = _gpu()
    dev = h.device()
    r = 64 if kind == "fp32" else 256
    g = synth.make_decode("bounds-app", 95, B=2, lens=[100, 70], r=r, H=4, d=32, k=8, M=16, paged=True,
                          dtype="fp32" if kind == "fp32" else "bf16")
    bt = g.block_table.copy()
    bt[1, 1] = g.num_pages + 3  # a page id past the pool
    max_pos = bt.shape[1] * 64
    # rows: two good ones, then bad sequence ids, bad positions and a bad page
    seq = np.array([0, 1, -1, 2, 0, 0, 1], dtype=np.int32)
    pos = np.array([5, 3, 4, 4, -5, max_pos, 64 + 7], dtype=np.int32)
    say(f"{kind}: append {len(seq)} rows, 5 of them outside the cache")
    tdt = torch.float32 if kind == "fp32" else torch.bfloat16
    rng = np.random.default_rng(1)
    rows = synth.round_bf16(rng.standard_normal((len(seq), r)).astype(np.float32))
    if kind == "fp8":
        pool = torch.zeros((g.num_pages, 64, r), dtype=torch.uint8, device=dev)
        scales = torch.zeros((g.num_pages, 64, r // 128), dtype=torch.float32, device=dev)
        cache = B.LatentCache(pool, h.i32(bt), h.i32(g.lens), scales)
    else:
        pool = torch.zeros((g.num_pages, 64, r), dtype=tdt, device=dev)
        cache = B.LatentCache(pool, h.i32(bt), h.i32(g.lens))
    if kind == "rope":
        B.append_latent_rope(cache, h.to_dev(rows, tdt), h.i32(seq), h.i32(pos), (16, 2))
    else:
        B.append_latent(cache, h.to_dev(rows, tdt), h.i32(seq), h.i32(pos))
    torch.cuda.synchronize()
    flat = pool.reshape(-1, r)
    written = torch.nonzero(flat.ne(0).any(dim=1)).flatten().cpu().numpy().tolist()
    want = sorted([int(bt[0, 0]) * 64 + 5, int(bt[1, 0]) * 64 + 3])
    assert sorted(written) == want, (written, want)
    if kind in ("bf16", "fp32"):  # copied bit for bit (FP8 and rotary rows are transformed)
        got = flat[int(bt[0, 0]) * 64 + 5].float().cpu().numpy()
        assert np.array_equal(got, rows[0])


def test_scoring_clamps_sequence_and_page_ids():
    """Query 2 names a sequence past the batch and sequence 1's block table
    holds page ids past the pool (in its unused tail and in a used page):
    the call completes, and query 0 (sequence 0, all indices valid) matches
    the oracle exactly as it does alone."""
    h = _gpu()
    g = synth.make_decode("bounds-score", 96, B=2, lens=[3000, 2000], r=256, H=64, d=128, k=256, M=512, paged=True)
    cache = h.build_cache(g)
    dev = h.device()
    bt = g.block_table.copy()
    bt[1, 5] = g.num_pages + 1000
    bt[1, -1] = -7
    cache.block_table = h.i32(bt)
    seq = h.i32(np.array([0, 1, 5], dtype=np.int32))
    pos = h.i32(np.array([2999, 1999, 100], dtype=np.int32))
    q = h.to_dev(np.concatenate([g.q[0], g.q[0][:1]]), torch.bfloat16)
    qt = B.absorb_query(q, h.to_dev(g.W[0], torch.bfloat16))
    w = torch.from_numpy(np.concatenate([g.w[0], g.w[0][:1]])).to(dev)
    say("scoring with out-of-range sequence and page ids")
    res = B.score_topk(cache, seq, pos, 3000, qt, w, g.k, keep_scores=True)
    torch.cuda.synchronize()
    o = oracle.full_layer(g.q[0], g.W[0], g.w[0], g.latent, g.qseq, g.qpos, g.lens, g.k, [0])[0]
    sc, idx, cnt = h.host(res.scores), h.host(res.idx), h.host(res.count)
    check_scores(sc[0, :3000], o.scores, "valid query beside garbage indices")
    check_topk(idx[0], int(cnt[0]), o.sel, o.scores, None, g.k, rms(o.scores), "valid query top-k")
    assert 0 <= int(cnt[2]) <= g.k and 0 <= int(cnt[1]) <= g.k

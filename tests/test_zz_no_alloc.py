"""GPU: li_score_topk_noalloc (scratch held by the library instead of a
workspace) gives the same results as li_score_topk, on two calls in a row,
the second smaller than the first; oversized calls are rejected."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from sparse_attention_token_absorb_amd import binding as B
from sparse_attention_token_absorb_amd import synth

pytestmark = pytest.mark.gpu


def say(msg: str) -> None:
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


def _gpu():
    import gpu_harness
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    return gpu_harness


def _case(h, g, l, k, k_inner):
    cache = h.build_cache(g)
    qs = h.Queries(g)
    qt = h.absorbed(g, l)
    w = h.head_weights(g, l)
    dev = h.device()
    Q = g.Q

    def outs(scores):
        o = B.TopK(torch.full((Q, k), -7, dtype=torch.int32, device=dev), torch.full((Q,), -7, dtype=torch.int32,
                                                                                      device=dev))
        if k_inner:
            o.idx_inner = torch.full((Q, k_inner), -7, dtype=torch.int32, device=dev)
            o.count_inner = torch.full((Q,), -7, dtype=torch.int32, device=dev)
        if scores:
            o.scores = torch.full((Q, qs.max_valid), float("nan"), device=dev)
        return o

    for with_scores in (True, False):
        ref = B.score_topk(cache, qs.seq, qs.pos, qs.max_valid, qt, w, k, k_inner=k_inner, out=outs(with_scores))
        got = B.score_topk_noalloc(cache, qs.seq, qs.pos, qs.max_valid, qt, w, k, outs(with_scores), k_inner=k_inner)
        torch.cuda.synchronize()
        assert torch.equal(ref.count, got.count)
        for i in range(Q):
            n = int(ref.count[i])
            assert set(ref.idx[i, :n].tolist()) == set(got.idx[i, :n].tolist()), (with_scores, i)
            assert torch.all(got.idx[i, n:] == -1)
        if k_inner:
            assert torch.equal(ref.count_inner, got.count_inner)
            for i in range(Q):
                n = int(ref.count_inner[i])
                assert set(ref.idx_inner[i, :n].tolist()) == set(got.idx_inner[i, :n].tolist())
        if with_scores:
            # identical kernels on identical inputs: bit-identical scores, untouched tails
            assert torch.equal(torch.nan_to_num(ref.scores, nan=-1.0), torch.nan_to_num(got.scores, nan=-1.0))


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    h = _gpu()
    big = synth.make_decode("noalloc-big", 91, B=4, lens=[131072, 70000, 131072, 9000], r=256, H=64, d=128, k=2048,
                            M=8192, G=1)
    say("first call: B=4, up to 131072 rows, HS-anchor budgets (k=8192 with nested 2048)")
    _case(h, big, 0, 8192, 2048)
    small = synth.make_decode("noalloc-small", 92, B=2, lens=[5000, 300], r=256, H=64, d=128, k=512, M=1024, G=1)
    say("second call: B=2, 5000 rows, k=512")
    _case(h, small, 0, 512, 0)


def test_noalloc_rejects_calls_beyond_its_scratch():
    h = _gpu()
    g = synth.make_decode("noalloc-huge", 93, B=1, lens=[64], r=256, H=64, d=128, k=64, M=64, G=1)
    cache = h.build_cache(g)
    dev = h.device()
    Q = 400  # 400 queries x 65536 rows of workspace scores: about 100 MiB
    seq = torch.zeros(Q, dtype=torch.int32, device=dev)
    pos = torch.zeros(Q, dtype=torch.int32, device=dev)
    qt = torch.zeros((Q, g.H, g.r), dtype=torch.bfloat16, device=dev)
    w = torch.ones((Q, g.H), dtype=torch.float32, device=dev)
    o = B.TopK(torch.empty((Q, 64), dtype=torch.int32, device=dev), torch.empty(Q, dtype=torch.int32, device=dev))
    big_cache = B.LatentCache(cache.pool, torch.zeros((1, 1024), dtype=torch.int32, device=dev), cache.seq_lens)
    with pytest.raises(B.LIError) as ei:
        B.score_topk_noalloc(big_cache, seq, pos, 65536, qt, w, 64, o)
    assert ei.value.status == B.LI_ERR_WORKSPACE and "scratch" in str(ei.value)

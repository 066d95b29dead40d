"""Graph capture and replay of the decode path (needs an MI355X).

The benchmark times captured graphs, so a captured sequence of library calls
must give what the same calls give eagerly, on every replay: the library
clears its histograms with a kernel (nothing a replay could skip), and the
outputs and the shared workspace are scribbled on by eager work between
replays here to show that each replay rewrites everything it reads.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from sparse_attention_token_absorb_amd import binding as B
from sparse_attention_token_absorb_amd import synth

pytestmark = pytest.mark.gpu


def say(msg: str) -> None:
    print(f"[graph] {msg}", flush=True)
    sys.stdout.flush()


def _sets(idx: torch.Tensor, cnt: torch.Tensor):
    i, c = idx.cpu().numpy(), cnt.cpu().numpy()
    return [frozenset(i[q, :c[q]].tolist()) for q in range(i.shape[0])], c.copy()


def test_graph_replays_match_eager():
    import gpu_harness as h
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    dev = h.device()
    g = synth.make_decode("graph", 80, B=3, lens=[20000, 9000, 30000], r=256, H=64, d=128, k=1024, M=4096)
    cache = h.build_cache(g)
    qs = h.Queries(g)
    N = qs.max_valid
    qt = [h.absorbed(g, l) for l in range(2)]
    w = [h.head_weights(g, l) for l in range(2)]
    Q = g.Q
    # FP8 copy of the same latent
    f8 = B.LatentCache(torch.zeros((g.num_pages, 64, g.r), dtype=torch.uint8, device=dev), h.i32(g.block_table),
                       h.i32(g.lens), torch.zeros((g.num_pages, 64, g.r // 128), dtype=torch.float32, device=dev))
    for b in range(g.B):
        n = int(g.lens[b])
        B.append_latent(f8, h.to_dev(g.latent[b][:n], torch.bfloat16), h.i32(np.full(n, b)), h.i32(np.arange(n)))
    f8q = B.absorb_query(h.to_dev(g.q[0], torch.bfloat16), h.to_dev(g.W[0], torch.bfloat16), fp8=True)

    ws = B.workspace(B.workspace_bytes(B.LI_OP_SCORE_TOPK, Q, N, 64, 256, g.M, 0), dev)
    ws_hs = B.workspace(B.workspace_bytes(B.LI_OP_HS_SELECT, Q, 0, 64, 256, g.k, g.M), dev)
    i32 = lambda *s: torch.empty(s, dtype=torch.int32, device=dev)
    full = B.TopK(i32(Q, g.k), i32(Q), scores=torch.empty((Q, N), dtype=torch.float32, device=dev))
    anchor = B.TopK(i32(Q, g.M), i32(Q), i32(Q, g.k), i32(Q))
    foll = B.TopK(i32(Q, g.k), i32(Q), scores=torch.empty((Q, g.M), dtype=torch.float32, device=dev))
    full8 = B.TopK(i32(Q, g.k), i32(Q), scores=torch.empty((Q, N), dtype=torch.float32, device=dev))
    other = B.TopK(i32(Q, g.k), i32(Q))

    def calls():
        B.score_topk(cache, qs.seq, qs.pos, N, qt[0], w[0], g.k, ws=ws, out=full)
        B.score_topk(cache, qs.seq, qs.pos, N, qt[0], w[0], g.M, k_inner=g.k, ws=ws, out=anchor)
        B.hs_select(cache, qs.seq, qs.pos, N, anchor.idx, anchor.count, qt[1], w[1], g.k, ws=ws_hs, out=foll)
        B.score_topk(f8, qs.seq, qs.pos, N, f8q, w[0], g.k, ws=ws, out=full8)

    def snapshot():
        torch.cuda.synchronize()
        return {"full": _sets(full.idx, full.count), "full_s": full.scores.cpu().numpy().copy(),
                "anchor": _sets(anchor.idx, anchor.count), "inner": _sets(anchor.idx_inner, anchor.count_inner),
                "anchor_raw": anchor.idx.cpu().numpy().copy(),
                "foll": _sets(foll.idx, foll.count), "foll_s": foll.scores.cpu().numpy().copy(),
                "full8": _sets(full8.idx, full8.count), "full8_s": full8.scores.cpu().numpy().copy()}

    stream = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(stream):
        calls()
    ref = snapshot()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        calls()
    torch.cuda.synchronize()
    for rep in range(4):
        say(f"replay {rep}")
        # eager work in between: another layer through the same workspaces,
        # and every output poisoned
        B.score_topk(cache, qs.seq, qs.pos, N, qt[1], w[1], g.k, ws=ws, out=other)
        B.hs_select(cache, qs.seq, qs.pos, N, other.idx, other.count, qt[0], w[0], g.k, ws=ws_hs)
        for t in (full.idx, full.count, anchor.idx, anchor.count, anchor.idx_inner, anchor.count_inner, foll.idx,
                  foll.count, full8.idx, full8.count):
            t.fill_(-7)
        for t in (full.scores, foll.scores, full8.scores):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        got = snapshot()
        for key, want in ref.items():
            if key == "anchor_raw":
                continue
            if key == "foll_s":
                # candidate slots follow the anchor's (set-like) output order:
                # compare each candidate position's score
                for q in range(Q):
                    n = int(ref["anchor"][1][q])
                    gm = dict(zip(got["anchor_raw"][q, :n].tolist(), got[key][q, :n].tolist()))
                    wm = dict(zip(ref["anchor_raw"][q, :n].tolist(), want[q, :n].tolist()))
                    assert gm == wm, f"replay {rep}: follower scores of query {q}"
            elif key.endswith("_s"):
                # scores: bit-identical wherever a valid row was scored
                for q in range(Q):
                    n = int(min(g.qpos[q] + 1, g.lens[g.qseq[q]]))
                    assert np.array_equal(got[key][q, :n], want[q, :n]), f"replay {rep}: {key} query {q}"
            else:
                assert got[key][0] == want[0] and np.array_equal(got[key][1], want[1]), f"replay {rep}: {key}"

"""Whole-model indexer step over a layer map.

LatentIndex (paperlayer.ai summary of arXiv:2610.04635): in the paper's
DeepSeek-V3.2 setting the first layer keeps its own indexer and the
remaining 60 layers form groups (§C.3: groups of 4, i.e. 15 groups; the
G = 8 variant is 7 groups of 8 and one of 4).  Within a group the anchor
caches the shared latent once per token (§3.1, §B.2) and every layer scores
it with its own absorbed query (full LatentIndex), or the anchor proposes
its top-M candidates and each follower rescores only those (hierarchical
selection, §3.2, §C.4).  The comparators are the native per-layer indexer on
every layer (DSA, §1, §B.3) and index reuse, where the followers take the
anchor's selection unchanged (IndexCache; HS with M = k selects the same
sets, §3.2).

This module only sequences calls of the library over the layer map (append,
query absorption or quantization, score + top-k, follower selection); every
arithmetic step runs in the library's kernels.  Nothing here allocates during
a step: queries, workspaces and outputs are allocated once at construction,
so a step can be captured in a HIP graph and replayed.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import torch

from . import binding as B

METHODS = ("dsa", "latentindex", "hs", "indexcache")


@dataclass(frozen=True)
class LayerMap:
    """Which layers keep their own indexer and how the others are grouped.

    independent: layer ids with a native per-layer indexer in every method.
    groups: tuples of layer ids, the anchor first; each group shares one
    latent cache.
    """
    n_layers: int
    independent: Tuple[int, ...]
    groups: Tuple[Tuple[int, ...], ...]

    @staticmethod
    def grouped(n_layers: int = 61, group: int = 4, independent: int = 1) -> "LayerMap":
        """The first `independent` layers on their own, the rest cut into
        consecutive groups of `group` layers; a shorter last group takes what
        is left (61 layers, G = 8: 7 groups of 8 and one of 4)."""
        if n_layers <= 0 or group <= 0 or not 0 <= independent <= n_layers:
            raise ValueError("n_layers, group > 0 and 0 <= independent <= n_layers")
        rest = list(range(independent, n_layers))
        groups = tuple(tuple(rest[i:i + group]) for i in range(0, len(rest), group))
        return LayerMap(n_layers, tuple(range(independent)), groups)

    def group_sizes(self) -> List[int]:
        return [len(g) for g in self.groups]


class IndexerModel:
    """The indexer of every layer of a model for one batch of decode queries.

    keys[l]     per-layer key cache (width d) of every layer that runs as a
                native indexer in some method: the independent layers, every
                layer for "dsa", the anchors for "indexcache".
    latents[g]  the shared latent cache (width r) of group g.
    q[l]        [Q][H][d] bf16 queries, W[l] [d][r] bf16 key decoders,
    w[l]        [Q][H] fp32 head weights.
    The caches are segmented FP8 when fp8 is set (uint8 pools with scales),
    else bf16.  k: selected rows per layer; M: HS candidates per query.
    max_valid: the largest causal prefix any step will be asked to score.
    keep_scores: keep every layer's scores in `out[l].scores` ([Q][max_valid]
    for full-prefix layers, [Q][M] for HS followers; entries past a query's
    rows are left untouched).
    """

    def __init__(self, lmap: LayerMap, keys: Dict[int, B.LatentCache], latents: Sequence[B.LatentCache],
                 q: Sequence[torch.Tensor], W: Sequence[torch.Tensor], w: Sequence[torch.Tensor], k: int, M: int,
                 max_valid: int, fp8: bool = False, keep_scores: bool = False):
        if len(latents) < len(lmap.groups):
            raise ValueError("one latent cache per group is needed")
        if not (len(q) == len(W) == len(w) == lmap.n_layers):
            raise ValueError("q, W and w need one entry per layer")
        self.lmap, self.keys, self.latents = lmap, dict(keys), list(latents)
        self.q, self.W, self.w = list(q), list(W), list(w)
        self.k, self.M, self.max_valid, self.fp8 = int(k), int(M), int(max_valid), bool(fp8)
        dev = self.q[0].device
        Q, H, d = (int(x) for x in self.q[0].shape)
        r = int(self.W[0].shape[1])
        self.Q, self.H, self.d, self.r = Q, H, d, r
        i32 = lambda *shape: torch.empty(shape, dtype=torch.int32, device=dev)
        f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
        nv = max(self.max_valid, 1)
        # absorbed (latent) and native (key) query operands of every layer
        if self.fp8:
            self.q_lat = [B.Fp8Query.empty(Q, H, r, dev) for _ in range(lmap.n_layers)]
            self.q_key = [B.Fp8Query.empty(Q, H, d, dev) for _ in range(lmap.n_layers)]
        else:
            self.q_lat = [torch.empty((Q, H, r), dtype=torch.bfloat16, device=dev) for _ in range(lmap.n_layers)]
            self.q_key = self.q  # a native bf16 indexer scores its keys with q as it is
        kmax = max(self.k, self.M)
        self.ws = B.workspace(max(B.workspace_bytes(B.LI_OP_SCORE_TOPK, Q, nv, H, max(r, d), kmax, 0),
                                  B.workspace_bytes(B.LI_OP_SCORE_TOPK_EXT_SCORES, Q, nv, H, max(r, d), kmax, 0)), dev)
        self.ws_hs = B.workspace(B.workspace_bytes(B.LI_OP_HS_SELECT, Q, 0, H, r, self.k, self.M), dev)
        self.out = [B.TopK(i32(Q, self.k), i32(Q), scores=f32(Q, nv) if keep_scores else None)
                    for _ in range(lmap.n_layers)]
        # HS anchors: top-M candidates with the anchor's own top-k nested
        self.out_anchor = [B.TopK(i32(Q, self.M), i32(Q), i32(Q, self.k), i32(Q),
                                  scores=f32(Q, nv) if keep_scores else None) for _ in lmap.groups]
        self.out_follower = [B.TopK(i32(Q, self.k), i32(Q), scores=f32(Q, self.M) if keep_scores else None)
                             for _ in range(lmap.n_layers)]
        self._have_cand = [False] * len(lmap.groups)

    # -- one layer's pieces ------------------------------------------------
    def _native(self, l: int, seq, pos, max_valid, new_key, new_seq, new_pos) -> B.TopK:
        """A native per-layer indexer: append the new key, prepare the query,
        score the layer's own keys and select."""
        cache = self.keys[l]
        if new_key is not None:
            B.append_latent(cache, new_key, new_seq, new_pos)
        if self.fp8:
            B.absorb_query(self.q[l], None, out=self.q_key[l], fp8=True)
        B.score_topk(cache, seq, pos, max_valid, self.q_key[l], self.w[l], self.k, ws=self.ws, out=self.out[l])
        return self.out[l]

    def _absorb(self, l: int) -> None:
        B.absorb_query(self.q[l], self.W[l], out=self.q_lat[l], fp8=self.fp8)

    # -- a whole step ------------------------------------------------------
    def step(self, method: str, seq: torch.Tensor, pos: torch.Tensor, max_valid: Optional[int] = None,
             new_keys: Optional[Dict[int, torch.Tensor]] = None,
             new_latents: Optional[Dict[int, torch.Tensor]] = None,
             new_seq: Optional[torch.Tensor] = None, new_pos: Optional[torch.Tensor] = None) -> Dict[int, B.TopK]:
        """One decode step of every layer's indexer under `method`.

        seq, pos: [Q] int32 queries (sequence and position).  new_keys[l] /
        new_latents[g]: rows [T][d] / [T][r] that layer l / group g's anchor
        appends first, at (new_seq, new_pos).  Returns each layer's selection
        (for an HS anchor its nested top-k; for an index-reuse follower the
        anchor's selection object itself).

        Under "hs", when max_valid <= M every query's candidate budget
        min(M, n) covers its whole prefix, so the candidates are every valid
        row and hierarchical selection is full LatentIndex on the group
        (§3.2): the group then runs as "latentindex" (same selections, no
        candidate list; candidates() refuses until an "hs" step with
        max_valid > M).
        """
        if method not in METHODS:
            raise ValueError(f"method must be one of {METHODS}")
        mv = self.max_valid if max_valid is None else int(max_valid)
        if mv > self.max_valid:
            raise ValueError("max_valid above the capacity the model was built for")
        nk = new_keys or {}
        nl = new_latents or {}
        sel: Dict[int, B.TopK] = {}
        for l in self.lmap.independent:
            sel[l] = self._native(l, seq, pos, mv, nk.get(l), new_seq, new_pos)
        for gi, layers in enumerate(self.lmap.groups):
            anchor = layers[0]
            if method == "dsa":
                for l in layers:
                    sel[l] = self._native(l, seq, pos, mv, nk.get(l), new_seq, new_pos)
                continue
            if method == "indexcache":
                a = self._native(anchor, seq, pos, mv, nk.get(anchor), new_seq, new_pos)
                for l in layers:
                    sel[l] = a
                continue
            lat = self.latents[gi]
            if gi in nl:
                B.append_latent(lat, nl[gi], new_seq, new_pos)
            full = method == "latentindex" or mv <= self.M
            if method == "hs":
                self._have_cand[gi] = not full
            for j, l in enumerate(layers):
                self._absorb(l)
                if full:
                    B.score_topk(lat, seq, pos, mv, self.q_lat[l], self.w[l], self.k, ws=self.ws, out=self.out[l])
                    sel[l] = self.out[l]
                elif j == 0:
                    oa = self.out_anchor[gi]
                    B.score_topk(lat, seq, pos, mv, self.q_lat[l], self.w[l], self.M, k_inner=self.k, ws=self.ws,
                                 out=oa)
                    sel[l] = B.TopK(oa.idx_inner, oa.count_inner, scores=oa.scores)
                else:
                    oa = self.out_anchor[gi]
                    B.hs_select(lat, seq, pos, mv, oa.idx, oa.count, self.q_lat[l], self.w[l], self.k, ws=self.ws_hs,
                                out=self.out_follower[l])
                    sel[l] = self.out_follower[l]
        return sel

    def candidates(self, group: int) -> B.TopK:
        """The HS anchor's top-M candidates of group `group` (after an "hs"
        step whose max_valid exceeded M; with a smaller bound the candidates
        were every valid row and no list was made)."""
        if not self._have_cand[group]:
            raise ValueError("no candidate list: the last hs step's budget M covered every row, or none ran")
        return self.out_anchor[group]

"""Helpers that put a synthetic workload on the GPU and run the HIP path.

Only marshalling: arrays from the seeded generator become device tensors,
and the library's entry points (through the binding) do all the work,
including writing the latent cache (the anchor's append).
"""
from __future__ import annotations

import numpy as np
import torch

from sparse_attention_token_absorb_amd import binding as B


def device() -> torch.device:
    return torch.device("cuda:0")


def torch_dtype(g) -> torch.dtype:
    return torch.bfloat16 if g.dtype == "bf16" else torch.float32


def to_dev(x: np.ndarray, dtype: torch.dtype, dev=None) -> torch.Tensor:
    """float32 numpy (already exact in `dtype`) -> device tensor of `dtype`."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(dtype).to(dev or device())


def i32(x, dev=None) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev or device())


def build_cache(g, rows_per_append: int | None = None, latent=None, r: int | None = None) -> B.LatentCache:
    """Zeroed page pool + block table; the rows go in through li_append_latent."""
    dev = device()
    latent = g.latent if latent is None else latent
    r = g.r if r is None else r
    dt = torch_dtype(g)
    pool = torch.zeros((max(g.num_pages, 1), 64, r), dtype=dt, device=dev)
    cache = B.LatentCache(pool, i32(g.block_table), i32(g.lens))
    for b in range(g.B):
        n = int(g.lens[b])
        step = n if rows_per_append is None else rows_per_append
        for s in range(0, n, max(step, 1)):
            e = min(n, s + step)
            B.append_latent(cache, to_dev(latent[b][s:e], dt), i32(np.full(e - s, b)), i32(np.arange(s, e)))
    return cache


class Queries:
    def __init__(self, g):
        self.seq = i32(g.qseq)
        self.pos = i32(g.qpos)
        lens = np.asarray(g.lens, dtype=np.int64)
        self.max_valid = int(max(min(int(p) + 1, int(lens[int(s)])) for s, p in zip(g.qseq, g.qpos))) if g.Q else 0


def absorbed(g, l: int) -> torch.Tensor:
    dt = torch_dtype(g)
    return B.absorb_query(to_dev(g.q[l], dt), to_dev(g.W[l], dt))


def head_weights(g, l: int) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(g.w[l], dtype=np.float32)).to(device())


def full_layer(g, cache, qs: Queries, l: int, k: int | None = None, k_inner: int = 0, keep_scores=True):
    qt = absorbed(g, l)
    return B.score_topk(cache, qs.seq, qs.pos, qs.max_valid, qt, head_weights(g, l), g.k if k is None else k,
                        k_inner=k_inner, keep_scores=keep_scores)


def hs_group(g, cache, qs: Queries, M: int | None = None, k: int | None = None, keep_scores=True):
    """Anchor top-M (with its own top-k nested) then every follower within the candidates."""
    M = g.M if M is None else M
    k = g.k if k is None else k
    anchor = full_layer(g, cache, qs, 0, k=M, k_inner=min(k, M), keep_scores=keep_scores)
    followers = []
    for l in range(1, g.G):
        qt = absorbed(g, l)
        followers.append(B.hs_select(cache, qs.seq, qs.pos, qs.max_valid, anchor.idx, anchor.count, qt,
                                     head_weights(g, l), k, keep_scores=keep_scores))
    return anchor, followers


def prefill_sample(Q: int, n: int = 64) -> list:
    """n evenly spaced query rows of a chunk, the first and the last included."""
    return sorted(set(np.linspace(0, Q - 1, n).round().astype(int).tolist()))


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()

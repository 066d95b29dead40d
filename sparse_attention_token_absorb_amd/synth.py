"""Seeded synthetic inputs for the LatentIndex indexer hot path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no absorption, scoring or selection).  Both the CPU
oracle and the GPU path consume what it returns, so it is the one piece of code
the two sides share.

Workload shapes follow the LatentIndex paper (paperlayer.ai summary):
  * a layer group of G = 4 layers with one shared latent cache (§3.1, §4.1);
  * a top-k budget of k = 2048 rows per query (§4.1), HS candidate budget 8192
    (§C.4), decode contexts of 8K-128K (§4.5);
  * an indexer with 64 heads of width 128 over a 256-wide latent.
The pages print no dataset items or worked inputs; every value here is drawn
from the distributions stated per configuration below.

Draw order (numpy PCG64, ``SeedSequence(seed).spawn``): latent Z, structure
U and V, heavy rows, heavy direction u, per-layer (q, W_dec, w), ragged
lengths, page permutation.  Values for bf16 configurations are rounded to
bfloat16 (round to nearest even) here, once, so both sides see the same bits.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

PAGE_SIZE = 64


# ----------------------------------------------------------------------------
# bfloat16 rounding (round to nearest, ties to even) on float32 bit patterns.
# ----------------------------------------------------------------------------
def round_bf16(x: np.ndarray) -> np.ndarray:
    """Return float32 values exactly representable in bfloat16 (RNE)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x).astype(np.float32)


@dataclass
class DecodeGroup:
    """One layer group at a decode step (or a chunk of prefill queries).

    latent[b] holds the logical rows 0..lens[b]-1 of sequence b (float32
    values, bf16-exact when dtype == "bf16").  Query i belongs to sequence
    qseq[i] at position qpos[i]; layer l has q[l] [Q][H][d], W[l] [d][r] and
    w[l] [Q][H].  keys_a[l][b] (optional) is the per-layer key cache
    [lens[b]][d] of the per-layer (DSA-style) baseline indexer: layer l's
    decoder applied to the latent rows, rounded once to the dtype.
    """
    name: str
    dtype: str
    H: int
    d: int
    r: int
    G: int
    k: int
    M: int
    lens: np.ndarray
    latent: List[np.ndarray]
    qseq: np.ndarray
    qpos: np.ndarray
    q: List[np.ndarray]
    W: List[np.ndarray]
    w: List[np.ndarray]
    heavy: List[np.ndarray] = field(default_factory=list)
    block_table: Optional[np.ndarray] = None
    num_pages: int = 0
    keys_a: Optional[List[List[np.ndarray]]] = None

    @property
    def B(self) -> int:
        return len(self.lens)

    @property
    def Q(self) -> int:
        return len(self.qseq)

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else np.ascontiguousarray(x)


def _paging(lens: np.ndarray, rng: Optional[np.random.Generator]):
    """Block table with a seeded permutation of physical pages (identity if rng is None)."""
    pages_per = [(int(n) + PAGE_SIZE - 1) // PAGE_SIZE for n in lens]
    total = int(sum(pages_per))
    phys = np.arange(total, dtype=np.int32) if rng is None else rng.permutation(total).astype(np.int32)
    max_pages = max(pages_per) if pages_per else 1
    bt = np.full((len(lens), max(max_pages, 1)), -1, dtype=np.int32)
    o = 0
    for b, p in enumerate(pages_per):
        bt[b, :p] = phys[o:o + p]
        o += p
    return bt, total


def _latent_rows(n: int, r: int, rng_z, rng_uv, rng_heavy, u: np.ndarray, heavy_frac: float,
                 n_heavy: Optional[int], structure: bool):
    z = rng_z.standard_normal((n, r), dtype=np.float32)
    if structure:
        U = rng_uv.standard_normal((n, 16), dtype=np.float32)
        V = (rng_uv.standard_normal((16, r), dtype=np.float32) * np.float32(1.0 / 4.0))
        z += np.float32(0.5) * (U @ V)
    nh = int(round(heavy_frac * n)) if n_heavy is None else n_heavy
    nh = min(nh, n)
    rows = np.sort(rng_heavy.choice(n, size=nh, replace=False)).astype(np.int64)
    z[rows] += np.float32(3.0) * u
    return z, rows


def make_decode(name: str, seed: int, *, B: int, lens, r: int, H: int, d: int, G: int = 4,
                k: int, M: int, dtype: str = "bf16", heavy_frac: float = 0.01,
                n_heavy: Optional[int] = None, structure: bool = True,
                w_dist: str = "softplus", paged: bool = True, keys_a: bool = False) -> DecodeGroup:
    """Decode-step group: one query per sequence at its last position."""
    ss = np.random.SeedSequence(seed)
    s_z, s_uv, s_heavy, s_u, s_layers, s_len, s_perm = ss.spawn(7)
    rng_len = np.random.Generator(np.random.PCG64(s_len))
    if lens is None:
        raise ValueError("lens required")
    if isinstance(lens, tuple):  # (lo, hi) inclusive range -> seeded ragged lengths
        lens = rng_len.integers(lens[0], lens[1] + 1, size=B)
    lens = np.asarray(lens, dtype=np.int64).reshape(B)
    rng_z = np.random.Generator(np.random.PCG64(s_z))
    rng_uv = np.random.Generator(np.random.PCG64(s_uv))
    rng_heavy = np.random.Generator(np.random.PCG64(s_heavy))
    rng_u = np.random.Generator(np.random.PCG64(s_u))
    u = rng_u.standard_normal(r, dtype=np.float32)
    latent, heavy = [], []
    for b in range(B):
        z, rows = _latent_rows(int(lens[b]), r, rng_z, rng_uv, rng_heavy, u, heavy_frac, n_heavy, structure)
        latent.append(_cast(z, dtype))
        heavy.append(rows)
    qs, Ws, ws, ka = [], [], [], []
    for ls in s_layers.spawn(G):
        rng = np.random.Generator(np.random.PCG64(ls))
        qs.append(_cast(rng.standard_normal((B, H, d), dtype=np.float32), dtype))
        Ws.append(_cast(rng.standard_normal((d, r), dtype=np.float32) * np.float32(1.0 / np.sqrt(r)), dtype))
        if w_dist == "softplus":
            wl = softplus(rng.standard_normal((B, H), dtype=np.float32))
        else:
            wl = rng.random((B, H), dtype=np.float32)
        ws.append(np.ascontiguousarray(wl, dtype=np.float32))
        if keys_a:
            # Per-layer key caches of the DSA-style baseline: the keys the layer
            # would cache natively for the same tokens, its decoder applied to
            # the latent rows (K_j = W_dec c_j, computed in float64 and rounded
            # once to the cache dtype), so the baseline and the latent path
            # score the same effective keys up to that one rounding.  These
            # keys are an input of the baseline (what it has cached), not a
            # step of either path; no random number is drawn for them.
            W64 = Ws[-1].astype(np.float64)
            ka.append([_cast(latent[b].astype(np.float64) @ W64.T, dtype) for b in range(B)])
    rng_perm = np.random.Generator(np.random.PCG64(s_perm)) if paged else None
    bt, npages = _paging(lens, rng_perm)
    return DecodeGroup(name=name, dtype=dtype, H=H, d=d, r=r, G=G, k=k, M=M, lens=lens.astype(np.int32),
                       latent=latent, qseq=np.arange(B, dtype=np.int32), qpos=(lens - 1).astype(np.int32),
                       q=qs, W=Ws, w=ws, heavy=heavy, block_table=bt, num_pages=npages,
                       keys_a=ka if keys_a else None)


def make_prefill(name: str, seed: int, *, N: int, Qn: int, r: int, H: int, d: int, G: int = 4,
                 k: int, dtype: str = "bf16", heavy_frac: float = 0.01) -> DecodeGroup:
    """Chunked prefill: the last Qn positions of an N-row cache, one sequence."""
    ss = np.random.SeedSequence(seed)
    s_z, s_uv, s_heavy, s_u, s_layers, s_len, s_perm = ss.spawn(7)
    rng_z = np.random.Generator(np.random.PCG64(s_z))
    rng_heavy = np.random.Generator(np.random.PCG64(s_heavy))
    rng_u = np.random.Generator(np.random.PCG64(s_u))
    u = rng_u.standard_normal(r, dtype=np.float32)
    z, rows = _latent_rows(N, r, rng_z, None, rng_heavy, u, heavy_frac, None, structure=False)
    qs, Ws, ws = [], [], []
    for ls in s_layers.spawn(G):
        rng = np.random.Generator(np.random.PCG64(ls))
        qs.append(_cast(rng.standard_normal((Qn, H, d), dtype=np.float32), dtype))
        Ws.append(_cast(rng.standard_normal((d, r), dtype=np.float32) * np.float32(1.0 / np.sqrt(r)), dtype))
        ws.append(softplus(rng.standard_normal((Qn, H), dtype=np.float32)))
    lens = np.array([N], dtype=np.int32)
    bt, npages = _paging(lens, None)
    return DecodeGroup(name=name, dtype=dtype, H=H, d=d, r=r, G=G, k=k, M=0, lens=lens,
                       latent=[_cast(z, dtype)], qseq=np.zeros(Qn, dtype=np.int32),
                       qpos=(N - Qn + np.arange(Qn)).astype(np.int32), q=qs, W=Ws, w=ws,
                       heavy=[rows], block_table=bt, num_pages=npages)


# ----------------------------------------------------------------------------
# The five workloads.  ``scale`` < 1 shrinks the row counts for quick runs
# while keeping every other property (shapes of heads, widths, budgets).
# ----------------------------------------------------------------------------
def tiny_fp32_n512(seed: int = 1) -> DecodeGroup:
    """Tiny fp32 group: N=512, r=64, H=4, d=32, k=64, M=128, 8 heavy rows."""
    return make_decode("tiny-fp32-N512", seed, B=1, lens=[512], r=64, H=4, d=32, k=64, M=128,
                       dtype="fp32", n_heavy=8, structure=False, w_dist="uniform", paged=False)


def decode_b1_n8192(seed: int = 2) -> DecodeGroup:
    """DSA-scale single decode: N=8192, H=64, d=128, r=256, bf16, k=2048."""
    return make_decode("decode-B1-N8192", seed, B=1, lens=[8192], r=256, H=64, d=128, k=2048, M=8192,
                       paged=False)


def ragged_paged_b16(seed: int = 3, lo: int = 16384, hi: int = 32768, B: int = 16) -> DecodeGroup:
    """Ragged paged HS decode: B=16, lens ~ U{16384..32768}, M=8192, k=2048."""
    return make_decode(f"hs-ragged-B{B}-N{lo}-{hi}", seed, B=B, lens=(lo, hi), r=256, H=64, d=128,
                       k=2048, M=8192, paged=True)


def long_context_b4(seed: int = 4, N: int = 131072, B: int = 4, keys_a: bool = True) -> DecodeGroup:
    """Long-context decode: B=4, N=131072, r=256 (plus [N][128] per-layer keys)."""
    return make_decode(f"decode-B{B}-N{N}", seed, B=B, lens=[N] * B, r=256, H=64, d=128, k=2048, M=8192,
                       paged=True, keys_a=keys_a)


def chunked_prefill_q4096(seed: int = 5, N: int = 65536, Qn: int = 4096) -> DecodeGroup:
    """Chunked prefill: 4096 queries at positions N-4096..N-1 of a 65536-row cache."""
    return make_prefill(f"prefill-Q{Qn}-N{N}", seed, N=N, Qn=Qn, r=256, H=64, d=128, k=2048)


# ----------------------------------------------------------------------------
# RoPE-compatible structured decoder (§A.2-§A.4): F rotary frequencies with S
# complex sources each, and a NoPE latent.  The native key is 2F rotary + d_nope
# NoPE wide; the latent 2SF rotary + r_nope NoPE wide.
# ----------------------------------------------------------------------------
@dataclass
class RopeGroup:
    """Per-layer structured decoders for one layer group.

    D[l] [F][S][2] decoder coefficients (re, im), Wn[l] [d_nope][r_nope] NoPE
    decoder, beta[l] [d_nope] NoPE output bias (fp32); F, S, base describe the
    latent's rotary part.  Values are bf16-exact except beta."""
    F: int
    S: int
    base: float
    d_nope: int
    r_nope: int
    D: List[np.ndarray]
    Wn: List[np.ndarray]
    beta: List[np.ndarray]

    @property
    def d_rope(self) -> int:
        return 2 * self.F

    @property
    def d(self) -> int:
        return 2 * self.F + self.d_nope

    @property
    def r(self) -> int:
        return 2 * self.S * self.F + self.r_nope


def make_rope(seed: int, *, G: int = 4, F: int = 32, S: int = 2, d_nope: int = 64, r_nope: int = 128,
              base: float = 10000.0, beta_scale: float = 0.5) -> RopeGroup:
    """Decoders: D ~ complex N(0, 1/S) per coefficient, Wn ~ N(0, 1/r_nope),
    beta ~ N(0, beta_scale^2); all but beta rounded to bf16."""
    ss = np.random.SeedSequence(seed)
    Ds, Wns, betas = [], [], []
    for ls in ss.spawn(G):
        rng = np.random.Generator(np.random.PCG64(ls))
        Ds.append(round_bf16(rng.standard_normal((F, S, 2), dtype=np.float32) * np.float32(1.0 / np.sqrt(2.0 * S))))
        Wns.append(round_bf16(rng.standard_normal((d_nope, r_nope), dtype=np.float32) *
                              np.float32(1.0 / np.sqrt(r_nope))))
        betas.append((rng.standard_normal(d_nope, dtype=np.float32) * np.float32(beta_scale)).astype(np.float32))
    return RopeGroup(F=F, S=S, base=base, d_nope=d_nope, r_nope=r_nope, D=Ds, Wn=Wns, beta=betas)

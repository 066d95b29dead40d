"""CPU oracle for the LatentIndex indexer hot path (fp64, plain loops).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only code allowed to import this package.  It
imports nothing from the GPU package and the GPU package imports nothing from
it; the two share only the seeded input generator.

The arithmetic lives in ``li_oracle.c`` (built with gcc into
``liboracle.so``); this module marshals numpy arrays in and composes the
per-layer steps into the two selection schemes of the LatentIndex paper
(paperlayer.ai summary of arXiv:2610.04635):

  O1 valid rows   a query at position p of a sequence with len rows scores
                  rows 0..min(p, len-1) (causal prefix, inclusive; §C.4 caps
                  budgets at the valid prefix)
  O2 absorb       qt = q W_dec                                 (§3.1, §B.2)
  O3 score        s(j) = sum_h w_h max(0, qt_h . c_j)          (§3.1, §B.2)
  O4 top-k        first min(k, n) of (score desc, position asc) (§3.1, §4.1, §C.4)
  O5 HS           anchor proposes its top-min(M, n); each follower rescores
                  only those and takes its own top-min(k, |cand|)  (§3.2, §C.4)
  O6 explicit     score through rebuilt keys K_j = W_dec c_j       (§1, §3.1)
  O8 counters     rows scored per query and group                  (§3.4, §B.3)
  O9 rope         rotate the latent's rotary sources by the native phase
                  of their position before caching                  (§A.2, §A.4)
  O10 absorb_rope structured absorption: per-frequency complex decoder
                  coefficients, dense NoPE decoder, output bias     (§A.2-§A.4)
  O11 explicit    scores through rebuilt post-RoPE native keys      (§3.1, §A.2)

Parity: every function here is pinned by the CPU tests (hand-derived worked
examples under tests/golden/, the absorption identity, brute-force selection
on tiny inputs, the HS reductions and the paper's closed forms).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "li_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)
_i64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile li_oracle.c with gcc (OpenMP) into liboracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", _SRC,
                               "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load(path: Optional[str] = None):
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _bind(lib):
    lib.lio_absorb.argtypes = [_dp, _dp, _i64, _i64, _i64, _i64, _dp]
    lib.lio_absorb.restype = None
    lib.lio_score.argtypes = [_dp, _dp, _dp, _dp, _ip, _i64, _i64, _i64, _dp]
    lib.lio_score.restype = None
    lib.lio_score_explicit.argtypes = [_dp, _dp, _dp, _dp, _i64, _i64, _i64, _i64, _dp]
    lib.lio_score_explicit.restype = None
    lib.lio_topk.argtypes = [_dp, _ip, _i64, _i64, _ip]
    lib.lio_topk.restype = _i64
    lib.lio_threads.argtypes = []
    lib.lio_threads.restype = ctypes.c_int
    u8 = ctypes.c_uint8
    _u8p = ctypes.POINTER(u8)
    _fp = ctypes.POINTER(ctypes.c_float)
    lib.lio_e4m3_decode.argtypes = [u8]
    lib.lio_e4m3_decode.restype = ctypes.c_double
    lib.lio_e4m3_encode.argtypes = [ctypes.c_float]
    lib.lio_e4m3_encode.restype = u8
    lib.lio_wht128.argtypes = [_fp]
    lib.lio_wht128.restype = None
    lib.lio_pow2_exponent.argtypes = [ctypes.c_float]
    lib.lio_pow2_exponent.restype = ctypes.c_int
    lib.lio_quantize_rows.argtypes = [_fp, _i64, _i64, _u8p, _fp]
    lib.lio_quantize_rows.restype = None
    lib.lio_score_fp8.argtypes = [_u8p, _fp, _dp, _dp, _u8p, _fp, _ip, _i64, _i64, _i64, _dp]
    lib.lio_score_fp8.restype = None
    lib.lio_rope_rotate.argtypes = [_dp, _ip, _i64, _i64, _i64, _i64, ctypes.c_double]
    lib.lio_rope_rotate.restype = None
    lib.lio_absorb_rope.argtypes = [_dp, _dp, _dp, _dp, _i64, _i64, _i64, _i64, _i64, _dp, _dp]
    lib.lio_absorb_rope.restype = None
    lib.lio_score_explicit_rope.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _ip, _i64, _i64, _i64, _i64, _i64, _i64,
                                            ctypes.c_double, _dp]
    lib.lio_score_explicit_rope.restype = None
    return lib


def use_library(path: Optional[str]) -> None:
    """Point the oracle at another build of li_oracle.c (None: the default)."""
    global _lib
    _lib = None if path is None else _load(path)


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: np.ndarray, t):
    return a.ctypes.data_as(t)


# ----------------------------------------------------------------------------
# Single steps
# ----------------------------------------------------------------------------
def valid_rows(pos: int, length: int) -> int:
    """O1: number of rows a query at ``pos`` scores in a ``length``-row sequence."""
    return int(max(0, min(int(pos) + 1, int(length))))


def absorb(q: np.ndarray, W: np.ndarray) -> np.ndarray:
    """O2: qt[..., h, t] = sum_e q[..., h, e] W[e, t]  (q [..., H, d], W [d, r])."""
    q = _f64(q)
    W = _f64(W)
    d, r = W.shape
    assert q.shape[-1] == d
    lead = q.shape[:-1]
    QH = int(np.prod(lead)) if lead else 1
    out = np.empty(lead + (r,), dtype=np.float64)
    _load().lio_absorb(_ptr(q, _dp), _ptr(W, _dp), QH, 1, d, r, _ptr(out, _dp))
    return out


def score(qt: np.ndarray, w: np.ndarray, C: np.ndarray, n: Optional[int] = None,
          rows: Optional[np.ndarray] = None, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """O3: scores of latent rows 0..n-1 (or of ``rows``) for one absorbed query.

    qt [H][r], w [H], C [*][r]; bias [H] (the absorbed decoder bias) or None.
    """
    qt = _f64(qt)
    w = _f64(w)
    C = _f64(C)
    H, r = qt.shape
    assert C.shape[1] == r and w.shape == (H,)
    bp = None
    if bias is not None:
        bias = _f64(bias)
        assert bias.shape == (H,)
        bp = _ptr(bias, _dp)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        assert rows.size == 0 or (rows.min() >= 0 and rows.max() < C.shape[0])
        m = rows.size
        rp = _ptr(rows, _ip)
    else:
        m = C.shape[0] if n is None else int(n)
        assert m <= C.shape[0]
        rp = None
    out = np.empty(m, dtype=np.float64)
    if m:
        _load().lio_score(_ptr(qt, _dp), _ptr(w, _dp), bp, _ptr(C, _dp), rp, m, H, r, _ptr(out, _dp))
    return out


def score_explicit(q: np.ndarray, W: Optional[np.ndarray], w: np.ndarray, C: np.ndarray,
                   n: Optional[int] = None) -> np.ndarray:
    """O6: scores through rebuilt per-layer keys K_j = W c_j (W=None: C are keys)."""
    q = _f64(q)
    w = _f64(w)
    C = _f64(C)
    H, d = q.shape
    r = C.shape[1]
    if W is not None:
        W = _f64(W)
        assert W.shape == (d, r)
    else:
        assert r == d
    m = C.shape[0] if n is None else int(n)
    out = np.empty(m, dtype=np.float64)
    if m:
        _load().lio_score_explicit(_ptr(q, _dp), None if W is None else _ptr(W, _dp), _ptr(w, _dp),
                                   _ptr(C, _dp), m, H, d, r, _ptr(out, _dp))
    return out


def topk(s: np.ndarray, K: int, pos: Optional[np.ndarray] = None) -> np.ndarray:
    """O4: positions of the first min(K, m) entries by (score desc, position asc)."""
    s = _f64(s)
    m = s.size
    K = max(0, min(int(K), m))
    out = np.empty(K, dtype=np.int32)
    pp = None
    if pos is not None:
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        assert pos.size == m
        pp = _ptr(pos, _ip)
    if K:
        got = _load().lio_topk(_ptr(s, _dp), pp, m, K, _ptr(out, _ip))
        if got != K:
            raise MemoryError("oracle top-k allocation failed")
    return out


# ----------------------------------------------------------------------------
# Segmented FP8 (reading of §A.2 / §B.2; see li_oracle.c)
# ----------------------------------------------------------------------------
_u8p = ctypes.POINTER(ctypes.c_uint8)
_fp = ctypes.POINTER(ctypes.c_float)
SEGMENT = 128


def e4m3_decode(codes) -> np.ndarray:
    """Values (fp64) of OCP E4M3 codes."""
    c = np.asarray(codes, dtype=np.uint8)
    L = _load()
    flat = np.array([L.lio_e4m3_decode(int(x)) for x in c.ravel()], dtype=np.float64)
    return flat.reshape(c.shape)


def e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3 codes of fp32 values (ties to even, saturating at 448)."""
    x = np.asarray(v, dtype=np.float32)
    L = _load()
    flat = np.array([L.lio_e4m3_encode(float(a)) for a in x.ravel()], dtype=np.uint8)
    return flat.reshape(x.shape)


def wht128(x) -> np.ndarray:
    """Orthonormal Walsh-Hadamard transform of one 128-vector, in fp32."""
    y = np.ascontiguousarray(x, dtype=np.float32).copy()
    assert y.shape == (SEGMENT,)
    _load().lio_wht128(_ptr(y, _fp))
    return y


def pow2_exponent(amax: float) -> int:
    """Smallest e with amax * 2^-e <= 448 (0 for amax = 0), clamped to [-120, 120]."""
    return int(_load().lio_pow2_exponent(float(np.float32(amax))))


def quantize_rows(x) -> tuple:
    """Rows [..., r] (fp32, r a multiple of 128) -> (codes [..., r] uint8,
    scales [..., r/128] fp32 powers of two)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    r = x.shape[-1]
    assert r % SEGMENT == 0
    lead = x.shape[:-1]
    rows = int(np.prod(lead)) if lead else 1
    codes = np.empty(lead + (r,), dtype=np.uint8)
    scales = np.empty(lead + (r // SEGMENT,), dtype=np.float32)
    if rows:
        _load().lio_quantize_rows(_ptr(x, _fp), rows, r, _ptr(codes, _u8p), _ptr(scales, _fp))
    return codes, scales


def score_fp8(qc, qs, w, cc, cs, n: Optional[int] = None, rows: Optional[np.ndarray] = None,
              bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Scores from FP8 operands: qc [H][r] codes, qs [H][r/128], w [H],
    cc [*][r] codes, cs [*][r/128]; rows 0..n-1 or the given ``rows``;
    bias [H] (the absorbed decoder bias, added before the ReLU) or None."""
    qc = np.ascontiguousarray(qc, dtype=np.uint8)
    qs = np.ascontiguousarray(qs, dtype=np.float32)
    w = _f64(w)
    cc = np.ascontiguousarray(cc, dtype=np.uint8)
    cs = np.ascontiguousarray(cs, dtype=np.float32)
    H, r = qc.shape
    assert cc.shape[1] == r and qs.shape == (H, r // SEGMENT) and cs.shape[1] == r // SEGMENT
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        assert rows.size == 0 or (rows.min() >= 0 and rows.max() < cc.shape[0])
        m = rows.size
        rp = _ptr(rows, _ip)
    else:
        m = cc.shape[0] if n is None else int(n)
        rp = None
    bp = None
    if bias is not None:
        bias = _f64(bias)
        assert bias.shape == (H,)
        bp = _ptr(bias, _dp)
    out = np.empty(m, dtype=np.float64)
    if m:
        _load().lio_score_fp8(_ptr(qc, _u8p), _ptr(qs, _fp), _ptr(w, _dp), bp, _ptr(cc, _u8p), _ptr(cs, _fp), rp, m,
                              H, r, _ptr(out, _dp))
    return out


def absorb_fp8(q: np.ndarray, W: np.ndarray) -> tuple:
    """Absorbed query in FP8: qt = q W (fp64, then rounded once to fp32),
    rotated and quantized per 128-element segment."""
    return quantize_rows(absorb(q, W).astype(np.float32))


# ----------------------------------------------------------------------------
# RoPE-compatible structured decoder (§A.2-§A.4; see li_oracle.c)
# ----------------------------------------------------------------------------
def rope_rotate(rows, pos, F: int, S: int, base: float = 10000.0) -> np.ndarray:
    """O9: latent rows [n][r] with their S*F source pairs rotated by the
    native rotary phase of their positions (fp64; a new array)."""
    x = _f64(rows).copy()
    n = x.shape[0] if x.ndim == 2 else 0
    r = x.shape[-1]
    assert 2 * S * F <= r
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    assert pos.shape == (n,)
    if n and S * F:
        _load().lio_rope_rotate(_ptr(x, _dp), _ptr(pos, _ip), n, r, F, S, float(base))
    return x


def absorb_rope(q, D, Wn, beta, F: int, S: int) -> tuple:
    """O10: structured absorption.  q [..., H, 2F + d_nope] (post-RoPE),
    D [F][S][2] decoder coefficients (re, im), Wn [d_nope][r_nope], beta
    [d_nope] -> (qt [..., H, 2SF + r_nope], bias [..., H])."""
    q = _f64(q)
    D = _f64(D).reshape(F, S, 2) if F * S else np.zeros((0,), dtype=np.float64)
    Wn = _f64(Wn)
    beta = _f64(beta)
    d_nope, r_nope = Wn.shape
    assert q.shape[-1] == 2 * F + d_nope and beta.shape == (d_nope,)
    lead = q.shape[:-1]
    QH = int(np.prod(lead)) if lead else 1
    qt = np.empty(lead + (2 * S * F + r_nope,), dtype=np.float64)
    b = np.empty(lead, dtype=np.float64)
    D = np.ascontiguousarray(D)
    _load().lio_absorb_rope(_ptr(q, _dp), _ptr(D, _dp), _ptr(Wn, _dp), _ptr(beta, _dp), QH, F, S, d_nope, r_nope,
                            _ptr(qt, _dp), _ptr(b, _dp))
    return qt, b


def score_explicit_rope(q, D, Wn, beta, w, C, pos, F: int, S: int, base: float = 10000.0) -> np.ndarray:
    """O11: scores of unrotated latent rows C [n][r] at positions ``pos``
    through the rebuilt post-RoPE native keys of the layer (q [H][d])."""
    q = _f64(q)
    w = _f64(w)
    C = _f64(C)
    D = np.ascontiguousarray(_f64(D).reshape(F, S, 2) if F * S else np.zeros((1,)))
    Wn = _f64(Wn)
    beta = _f64(beta)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    H = q.shape[0]
    d_nope, r_nope = Wn.shape
    n = C.shape[0]
    assert q.shape == (H, 2 * F + d_nope) and C.shape[1] == 2 * S * F + r_nope and pos.shape == (n,)
    out = np.empty(n, dtype=np.float64)
    if n:
        _load().lio_score_explicit_rope(_ptr(q, _dp), _ptr(D, _dp), _ptr(Wn, _dp), _ptr(beta, _dp), _ptr(w, _dp),
                                        _ptr(C, _dp), _ptr(pos, _ip), n, H, F, S, d_nope, r_nope, float(base),
                                        _ptr(out, _dp))
    return out


# ----------------------------------------------------------------------------
# Group compositions
# ----------------------------------------------------------------------------
class LayerResult:
    __slots__ = ("scores", "sel", "cand", "cand_scores")

    def __init__(self, scores=None, sel=None, cand=None, cand_scores=None):
        self.scores = scores
        self.sel = sel
        self.cand = cand
        self.cand_scores = cand_scores


def full_layer(q_l, W_l, w_l, latents: Sequence[np.ndarray], qseq, qpos, lens, k: int,
               queries: Optional[Sequence[int]] = None) -> List[LayerResult]:
    """Full LatentIndex for one layer: absorb, score the valid prefix, top-k."""
    out = []
    idx = range(len(qseq)) if queries is None else queries
    for i in idx:
        b = int(qseq[i])
        n = valid_rows(qpos[i], lens[b])
        qt = absorb(q_l[i], W_l)
        s = score(qt, w_l[i], latents[b], n)
        out.append(LayerResult(scores=s, sel=topk(s, min(k, n))))
    return out


def baseline_layer(q_l, w_l, keys: Sequence[np.ndarray], qseq, qpos, lens, k: int) -> List[LayerResult]:
    """Per-layer indexer on its own key cache (no decoder): explicit-key scoring + top-k."""
    out = []
    for i in range(len(qseq)):
        b = int(qseq[i])
        n = valid_rows(qpos[i], lens[b])
        s = score_explicit(q_l[i], None, w_l[i], keys[b], n)
        out.append(LayerResult(scores=s, sel=topk(s, min(k, n))))
    return out


def hs_group(q, W, w, latents, qseq, qpos, lens, k: int, M: int) -> List[List[LayerResult]]:
    """O5: hierarchical selection over a group; layer 0 is the anchor.

    Anchor: cand = top-min(M, n) of its full-prefix scores, sel = top-min(k, n).
    Follower l >= 1: scores only cand, sel = top-min(k, |cand|) of those, as
    absolute positions.
    """
    G = len(q)
    res: List[List[LayerResult]] = [[] for _ in range(G)]
    for i in range(len(qseq)):
        b = int(qseq[i])
        n = valid_rows(qpos[i], lens[b])
        qt0 = absorb(q[0][i], W[0])
        s0 = score(qt0, w[0][i], latents[b], n)
        cand = topk(s0, min(M, n))
        res[0].append(LayerResult(scores=s0, sel=topk(s0, min(k, n)), cand=cand))
        for l in range(1, G):
            qt = absorb(q[l][i], W[l])
            cs = score(qt, w[l][i], latents[b], rows=cand)
            sel = topk(cs, min(k, cand.size), pos=cand)
            res[l].append(LayerResult(scores=None, sel=sel, cand=cand, cand_scores=cs))
    return res


# ----------------------------------------------------------------------------
# Closed forms (§3.4, §B.1, §B.3)
# ----------------------------------------------------------------------------
def rows_scored_full(n: int, G: int) -> int:
    """O8: every layer of the group scores the full valid prefix."""
    return G * n


def rows_scored_hs(n: int, cand_size: int, G: int) -> int:
    """O8: the anchor scores n rows, each follower scores its candidate set."""
    return n + (G - 1) * cand_size


def model_positions_hs(L: int, independent: int, groups: int, G: int, M: int) -> int:
    """Scored positions per decode query over a whole model under HS."""
    return independent * L + groups * (L + (G - 1) * min(M, L))


def storage_bytes_per_token(n_layers: int, groups: int, G: int, key_bytes: int, latent_bytes: int):
    """Logical indexer-cache bytes per token: (per-layer keys, grouped latents).

    The native indexer keeps one key per layer; the grouped layout keeps one
    key for each independent layer plus one latent per group.
    """
    independent = n_layers - groups * G
    return n_layers * key_bytes, independent * key_bytes + groups * latent_bytes


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use in this process."""
    return int(_load().lio_threads())

"""Thin Python binding of liblatentindex (ctypes over the C ABI).

Argument marshalling only: tensors are checked for device, dtype and layout,
outputs and workspaces are allocated with torch, and every call goes straight
to the C entry point of the same name on the current HIP stream.  Every step
of the computation runs in the library's HIP kernels.  There is no fallback:
if the library is missing or fails to load, ``lib()`` raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblatentindex.so")

LI_OK, LI_ERR_NULL, LI_ERR_SHAPE, LI_ERR_UNSUPPORTED, LI_ERR_WORKSPACE, LI_ERR_HIP = range(6)
LI_BF16, LI_FP32, LI_FP8 = 0, 1, 2
LI_OP_SCORE_TOPK, LI_OP_HS_SELECT, LI_OP_SCORE_TOPK_EXT_SCORES = 0, 1, 2
PAGE_SIZE = 64
EXPORTED = ["li_append_latent", "li_append_latent_rope", "li_rope_decoder", "li_query_bias", "li_absorb_query",
            "li_score_topk", "li_score_topk_noalloc", "li_hs_select", "li_workspace_bytes", "li_fp8_query_bytes", "li_fp8_query_scale_offset",
            "li_timing_enable", "li_timing_read", "li_fused_filter", "li_phase_records", "li_status_str", "li_last_error",
            "li_abi_version"]
(LI_KERNEL_SCORE_DECODE, LI_KERNEL_SCORE_PREFILL, LI_KERNEL_SCORE_GATHER, LI_KERNEL_SELECT, LI_KERNEL_ABSORB,
 LI_KERNEL_APPEND) = range(6)


class LIError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({_status_name(status)}): {detail}")
        self.status = status


class _Cache(ctypes.Structure):
    _fields_ = [("pool", ctypes.c_void_p), ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("max_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("r", ctypes.c_int32), ("dtype", ctypes.c_int),
                ("scales", ctypes.c_void_p)]


class _Rope(ctypes.Structure):
    _fields_ = [("freqs", ctypes.c_int32), ("sources", ctypes.c_int32), ("base", ctypes.c_double)]


class _Queries(ctypes.Structure):
    _fields_ = [("seq", ctypes.c_void_p), ("pos", ctypes.c_void_p), ("Q", ctypes.c_int32),
                ("max_valid", ctypes.c_int32)]


_lib = None


def lib():
    """Load liblatentindex.so (built in-tree).  Raises if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run python -m sparse_attention_token_absorb_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        cp, qp = ctypes.POINTER(_Cache), ctypes.POINTER(_Queries)
        L.li_append_latent.argtypes = [cp, vp, vp, vp, i32, vp]
        rp = ctypes.POINTER(_Rope)
        L.li_append_latent_rope.argtypes = [cp, vp, vp, vp, i32, rp, vp]
        L.li_rope_decoder.argtypes = [vp, vp, rp, i32, i32, vp, ctypes.c_int, vp]
        L.li_query_bias.argtypes = [vp, vp, i32, i32, i32, i32, vp, ctypes.c_int, vp]
        L.li_absorb_query.argtypes = [vp, vp, vp, i32, i32, i32, i32, ctypes.c_int, vp]
        L.li_score_topk.argtypes = [cp, qp, vp, vp, vp, i32, i32, vp, vp, i32, vp, vp, vp, i64, vp, sz, vp]
        L.li_score_topk_noalloc.argtypes = [cp, qp, vp, vp, vp, i32, i32, vp, vp, i32, vp, vp, vp, i64, vp]
        L.li_hs_select.argtypes = [cp, qp, vp, vp, i32, vp, vp, vp, i32, i32, vp, vp, vp, vp, sz, vp]
        L.li_workspace_bytes.argtypes = [ctypes.c_int, i32, i32, i32, i32, i32, i32]
        L.li_workspace_bytes.restype = sz
        for f in ("li_fp8_query_bytes", "li_fp8_query_scale_offset"):
            getattr(L, f).argtypes = [i32, i32, i32]
            getattr(L, f).restype = sz
        L.li_status_str.argtypes = [ctypes.c_int]
        L.li_status_str.restype = ctypes.c_char_p
        L.li_last_error.argtypes = []
        L.li_last_error.restype = ctypes.c_char_p
        L.li_abi_version.restype = i32
        L.li_timing_enable.argtypes = [ctypes.c_int]
        L.li_timing_enable.restype = ctypes.c_int
        L.li_timing_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
        L.li_timing_read.restype = ctypes.c_int
        L.li_fused_filter.argtypes = [ctypes.c_int]
        L.li_fused_filter.restype = ctypes.c_int
        L.li_phase_records.argtypes = [ctypes.c_int, vp, sz]
        L.li_phase_records.restype = ctypes.c_int
        for f in ("li_append_latent", "li_absorb_query", "li_score_topk", "li_hs_select"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _status_name(s: int) -> str:
    try:
        return lib().li_status_str(s).decode()
    except Exception:  # library not loadable: still give a readable message
        return str(s)


def _check(status: int, where: str) -> None:
    if status != LI_OK:
        raise LIError(status, where, lib().li_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, device=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _li_dtype(dt) -> int:
    if dt == torch.bfloat16:
        return LI_BF16
    if dt == torch.float32:
        return LI_FP32
    raise TypeError(f"unsupported dtype {dt} (bfloat16 or float32)")


@dataclass
class LatentCache:
    """Paged shared latent cache of one layer group (caller-owned tensors).

    pool [num_pages][64][r] (bf16 or fp32; uint8 E4M3 codes for a segmented
    FP8 cache, which then needs scales [num_pages][64][r/128] float32),
    block_table [batch][max_pages] int32, seq_lens [batch] int32.
    """
    pool: torch.Tensor
    block_table: torch.Tensor
    seq_lens: torch.Tensor
    scales: Optional[torch.Tensor] = None

    def __post_init__(self):
        if self.pool.dim() != 3 or self.pool.shape[1] != PAGE_SIZE:
            raise ValueError("pool must be [num_pages][64][r]")
        _need(self.pool, "pool", self.pool.dtype)
        dev = self.pool.device
        if self.pool.dtype == torch.uint8:
            if self.scales is None:
                raise ValueError("an FP8 cache needs scales [num_pages][64][r/128]")
            _need(self.scales, "scales", torch.float32, dev,
                  (self.pool.shape[0], PAGE_SIZE, self.pool.shape[2] // 128))
        else:
            _li_dtype(self.pool.dtype)
        _need(self.block_table, "block_table", torch.int32, dev)
        _need(self.seq_lens, "seq_lens", torch.int32, dev)
        if self.block_table.dim() != 2 or self.seq_lens.shape != (self.block_table.shape[0],):
            raise ValueError("block_table must be [batch][max_pages] and seq_lens [batch]")

    @property
    def fp8(self) -> bool:
        return self.pool.dtype == torch.uint8

    @property
    def device(self):
        return self.pool.device

    @property
    def r(self) -> int:
        return int(self.pool.shape[2])

    @property
    def dtype(self):
        return self.pool.dtype

    def desc(self) -> _Cache:
        return _Cache(self.pool.data_ptr(), self.block_table.data_ptr(), self.seq_lens.data_ptr(),
                      int(self.block_table.shape[0]), int(self.block_table.shape[1]), PAGE_SIZE,
                      int(self.pool.shape[0]), self.r, LI_FP8 if self.fp8 else _li_dtype(self.pool.dtype),
                      self.scales.data_ptr() if self.fp8 else None)


class Fp8Query:
    """Absorbed queries in segmented FP8: one uint8 buffer holding the codes
    [Q][H][r] and, at li_fp8_query_scale_offset, the scales [Q][H][r/128]."""

    def __init__(self, buf: torch.Tensor, Q: int, H: int, r: int):
        self.buf, self.Q, self.H, self.r = buf, Q, H, r

    @staticmethod
    def nbytes(Q: int, H: int, r: int) -> int:
        return int(lib().li_fp8_query_bytes(Q, H, r))

    @staticmethod
    def empty(Q: int, H: int, r: int, device) -> "Fp8Query":
        return Fp8Query(torch.empty(max(Fp8Query.nbytes(Q, H, r), 1), dtype=torch.uint8, device=device), Q, H, r)

    def codes(self) -> torch.Tensor:
        return self.buf[:self.Q * self.H * self.r].view(self.Q, self.H, self.r)

    def scales(self) -> torch.Tensor:
        off = int(lib().li_fp8_query_scale_offset(self.Q, self.H, self.r))
        n = self.Q * self.H * (self.r // 128)
        return self.buf[off:off + 4 * n].view(torch.float32).view(self.Q, self.H, self.r // 128)


def _queries(cache: LatentCache, seq: torch.Tensor, pos: torch.Tensor, max_valid: int) -> _Queries:
    _need(seq, "seq", torch.int32, cache.device)
    _need(pos, "pos", torch.int32, cache.device)
    if seq.dim() != 1 or pos.shape != seq.shape:
        raise ValueError("seq and pos must be [Q]")
    return _Queries(seq.data_ptr(), pos.data_ptr(), int(seq.shape[0]), int(max_valid))


def timing_enable(on: bool) -> None:
    """li_timing_enable: bracket every kernel-class launch with HIP events."""
    _check(lib().li_timing_enable(1 if on else 0), "li_timing_enable")


FUSED_FILTER_OFF, FUSED_FILTER_ON, FUSED_FILTER_FALLBACK = 0, 1, 2


def fused_filter(mode: int) -> None:
    """li_fused_filter: where the long-row selection's filter pass runs
    (0: its own kernel, 1: inside the decode scoring kernel, 2: as 1 with a
    wait that always runs out, so the final kernel's fallback runs)."""
    _check(lib().li_fused_filter(int(mode)), "li_fused_filter")


def timing_read(kernel_class: int) -> Tuple[float, int]:
    """li_timing_read: (summed ms, launches) of one class since the last read."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    _check(lib().li_timing_read(kernel_class, ctypes.byref(ms), ctypes.byref(n)), "li_timing_read")
    return float(ms.value), int(n.value)


LI_PHASE_SCORE_DECODE_BF16, LI_PHASE_SCORE_DECODE_FP8 = 0, 1
PHASE_RECORDS, PHASE_WORDS = 16384, 8


def phase_clear(kernel: int) -> None:
    """li_phase_records(kernel, NULL, 0): zero one decode kernel's phase records
    (instrumented "phases" build only; LIError otherwise)."""
    _check(lib().li_phase_records(kernel, None, 0), "li_phase_records")


def phase_records(kernel: int):
    """li_phase_records: the phase records as a [16384, 8] uint64 numpy array."""
    import numpy as np
    buf = np.zeros((PHASE_RECORDS, PHASE_WORDS), dtype=np.uint64)
    _check(lib().li_phase_records(kernel, buf.ctypes.data_as(ctypes.c_void_p), buf.nbytes), "li_phase_records")
    return buf


def workspace_bytes(op: int, Q: int, max_valid: int, H: int, r: int, k: int, M: int = 0) -> int:
    return int(lib().li_workspace_bytes(op, Q, max_valid, H, r, k, M))


def workspace(nbytes: int, device) -> torch.Tensor:
    """A workspace of nbytes, zero-filled: its leading region must be zero
    before its first use (li_workspace_bytes), and every call leaves it so."""
    return torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=device)


def _workspace(device, nbytes: int, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is None:
        return workspace(nbytes, device)
    _need(ws, "ws", torch.uint8, device)
    return ws


def append_latent(cache: LatentCache, rows: torch.Tensor, seq: torch.Tensor, pos: torch.Tensor) -> None:
    """li_append_latent: copy rows [T][r] into the pool at (seq[t], pos[t])
    (bf16 rows, rotated and quantized, for an FP8 cache)."""
    _need(rows, "rows", torch.bfloat16 if cache.fp8 else cache.dtype, cache.device)
    _need(seq, "seq", torch.int32, cache.device)
    _need(pos, "pos", torch.int32, cache.device)
    T = int(rows.shape[0])
    if rows.dim() != 2 or rows.shape[1] != cache.r or seq.shape != (T,) or pos.shape != (T,):
        raise ValueError("rows must be [T][r], seq and pos [T]")
    c = cache.desc()
    _check(lib().li_append_latent(ctypes.byref(c), _ptr(rows), _ptr(seq), _ptr(pos), T, _stream(cache.device)),
           "li_append_latent")


def _rope(rope) -> _Rope:
    F, S = int(rope[0]), int(rope[1])
    base = float(rope[2]) if len(rope) > 2 else 10000.0
    return _Rope(F, S, base)


def append_latent_rope(cache: LatentCache, rows: torch.Tensor, seq: torch.Tensor, pos: torch.Tensor, rope) -> None:
    """li_append_latent_rope: rows [T][r] with unrotated rotary sources;
    rope = (freqs, sources[, base])."""
    _need(rows, "rows", torch.bfloat16 if cache.fp8 else cache.dtype, cache.device)
    _need(seq, "seq", torch.int32, cache.device)
    _need(pos, "pos", torch.int32, cache.device)
    T = int(rows.shape[0])
    if rows.dim() != 2 or rows.shape[1] != cache.r or seq.shape != (T,) or pos.shape != (T,):
        raise ValueError("rows must be [T][r], seq and pos [T]")
    c = cache.desc()
    rd = _rope(rope)
    _check(lib().li_append_latent_rope(ctypes.byref(c), _ptr(rows), _ptr(seq), _ptr(pos), T, ctypes.byref(rd),
                                       _stream(cache.device)), "li_append_latent_rope")


def rope_decoder(D: torch.Tensor, w_nope: torch.Tensor, rope, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """li_rope_decoder: D [F][S][2], w_nope [d_nope][r_nope] (bf16 or fp32)
    -> the dense decoder w_dec [2F + d_nope][2SF + r_nope]."""
    dt = _li_dtype(D.dtype)
    F, S = int(rope[0]), int(rope[1])
    _need(D, "D", D.dtype, D.device, (F, S, 2))
    _need(w_nope, "w_nope", D.dtype, D.device)
    if w_nope.dim() != 2:
        raise ValueError("w_nope must be [d_nope][r_nope]")
    d_nope, r_nope = (int(x) for x in w_nope.shape)
    shape = (2 * F + d_nope, 2 * S * F + r_nope)
    if out is None:
        out = torch.empty(shape, dtype=D.dtype, device=D.device)
    _need(out, "w_dec", D.dtype, D.device, shape)
    rd = _rope(rope)
    _check(lib().li_rope_decoder(_ptr(D), _ptr(w_nope), ctypes.byref(rd), d_nope, r_nope, _ptr(out), dt,
                                 _stream(D.device)), "li_rope_decoder")
    return out


def query_bias(q: torch.Tensor, beta: torch.Tensor, d_rope: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """li_query_bias: q [Q][H][d] (bf16 or fp32), beta [d - d_rope] fp32 -> bias [Q][H] fp32."""
    dt = _li_dtype(q.dtype)
    _need(q, "q", q.dtype, q.device)
    if q.dim() != 3:
        raise ValueError("q must be [Q][H][d]")
    Q, H, d = (int(x) for x in q.shape)
    _need(beta, "beta", torch.float32, q.device, (d - d_rope,))
    if out is None:
        out = torch.empty((Q, H), dtype=torch.float32, device=q.device)
    _need(out, "bias", torch.float32, q.device, (Q, H))
    _check(lib().li_query_bias(_ptr(q), _ptr(beta), Q, H, d, d_rope, _ptr(out), dt, _stream(q.device)),
           "li_query_bias")
    return out


def absorb_query(q: torch.Tensor, w_dec: Optional[torch.Tensor], out=None, fp8: bool = False):
    """li_absorb_query: q [Q][H][d] x W_dec [d][r] -> q_tilde [Q][H][r]
    (an Fp8Query with fp8=True: bf16 inputs, rotated and quantized output;
    with fp8=True, w_dec None quantizes q itself, r = d)."""
    dev = q.device
    _need(q, "q", q.dtype, dev)
    dt = _li_dtype(q.dtype)
    if w_dec is None:
        if not fp8:
            raise ValueError("w_dec may be None only with fp8=True")
        if q.dim() != 3:
            raise ValueError("q must be [Q][H][d]")
        r = int(q.shape[2])
    else:
        _need(w_dec, "w_dec", q.dtype, dev)
        if q.dim() != 3 or w_dec.dim() != 2 or w_dec.shape[0] != q.shape[2]:
            raise ValueError("q must be [Q][H][d] and w_dec [d][r]")
        r = int(w_dec.shape[1])
    Q, H, d = (int(x) for x in q.shape)
    if fp8:
        if q.dtype != torch.bfloat16:
            raise TypeError("FP8 absorption takes bf16 q and w_dec")
        if out is None:
            out = Fp8Query.empty(Q, H, r, dev)
        if not isinstance(out, Fp8Query) or (out.Q, out.H, out.r) != (Q, H, r):
            raise ValueError("out must be an Fp8Query of the same shape")
        _need(out.buf, "out", torch.uint8, dev)
        if out.buf.numel() < Fp8Query.nbytes(Q, H, r):
            raise ValueError("FP8 query buffer too small")
        _check(lib().li_absorb_query(_ptr(q), _ptr(w_dec), _ptr(out.buf), Q, H, d, r, LI_FP8, _stream(dev)),
               "li_absorb_query")
        return out
    if out is None:
        out = torch.empty((Q, H, r), dtype=q.dtype, device=dev)
    _need(out, "out", q.dtype, dev, (Q, H, r))
    _check(lib().li_absorb_query(_ptr(q), _ptr(w_dec), _ptr(out), Q, H, d, r, dt, _stream(dev)), "li_absorb_query")
    return out


def _query_operand(cache: LatentCache, q_tilde, Q: int):
    """(H, device buffer) of the absorbed queries for this cache."""
    if cache.fp8:
        if not isinstance(q_tilde, Fp8Query) or q_tilde.Q != Q or q_tilde.r != cache.r:
            raise ValueError("an FP8 cache is scored with the Fp8Query of absorb_query(..., fp8=True)")
        _need(q_tilde.buf, "q_tilde", torch.uint8, cache.device)
        return q_tilde.H, q_tilde.buf
    _need(q_tilde, "q_tilde", cache.dtype, cache.device)
    if q_tilde.dim() != 3 or q_tilde.shape[0] != Q or q_tilde.shape[2] != cache.r:
        raise ValueError("q_tilde must be [Q][H][r]")
    return int(q_tilde.shape[1]), q_tilde


class TopK:
    """Outputs of score_topk / hs_select (device tensors)."""

    def __init__(self, idx, count, idx_inner=None, count_inner=None, scores=None):
        self.idx = idx
        self.count = count
        self.idx_inner = idx_inner
        self.count_inner = count_inner
        self.scores = scores


def topk_out_problem(out: TopK, Q: int, k: int, k_inner: int, max_valid: int) -> Optional[str]:
    """Why the output buffers of a score_topk call do not fit what the
    kernels write (dtype and shape; device placement is checked apart), or
    None when they do.  A buffer that is too small would be written past."""
    need = [("idx", out.idx, (Q, k)), ("count", out.count, (Q,))]
    if k_inner:
        if out.idx_inner is None or out.count_inner is None:
            return "k_inner > 0 needs idx_inner [Q][k_inner] and count_inner [Q]"
        need += [("idx_inner", out.idx_inner, (Q, k_inner)), ("count_inner", out.count_inner, (Q,))]
    for name, t, shape in need:
        if not isinstance(t, torch.Tensor):
            return f"{name} must be a torch tensor"
        if t.dtype != torch.int32:
            return f"{name} must be int32 (got {t.dtype})"
        if tuple(t.shape) != shape:
            return f"{name} has shape {tuple(t.shape)}, expected {shape}"
    if out.scores is not None:
        t = out.scores
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32:
            return "scores must be a float32 tensor"
        if t.dim() != 2 or t.shape[0] != Q or t.shape[1] < max(max_valid, 1):
            return f"scores must be [Q={Q}][ld >= {max(max_valid, 1)}], got {tuple(t.shape)}"
    return None


def _check_topk_out(out: TopK, Q: int, k: int, k_inner: int, max_valid: int, dev) -> None:
    """Every output buffer of a score_topk call has the shape the kernels write."""
    problem = topk_out_problem(out, Q, k, k_inner, max_valid)
    if problem:
        raise ValueError(problem)
    for name, t in (("idx", out.idx), ("count", out.count), ("idx_inner", out.idx_inner),
                    ("count_inner", out.count_inner), ("scores", out.scores)):
        if t is not None:
            _need(t, name, t.dtype, dev)


def score_topk(cache: LatentCache, seq: torch.Tensor, pos: torch.Tensor, max_valid: int, q_tilde: torch.Tensor,
               w: torch.Tensor, k: int, k_inner: int = 0, keep_scores: bool = False,
               ws: Optional[torch.Tensor] = None, out: Optional[TopK] = None,
               bias: Optional[torch.Tensor] = None) -> TopK:
    """li_score_topk: score every valid row and take the top-k (+ nested top-k_inner)."""
    dev = cache.device
    qs = _queries(cache, seq, pos, max_valid)
    Q = qs.Q
    H, qbuf = _query_operand(cache, q_tilde, Q)
    _need(w, "w", torch.float32, dev, (Q, H))
    if bias is not None:
        _need(bias, "bias", torch.float32, dev, (Q, H))
    if out is None:
        out = TopK(torch.empty((Q, k), dtype=torch.int32, device=dev), torch.empty(Q, dtype=torch.int32, device=dev))
        if k_inner:
            out.idx_inner = torch.empty((Q, k_inner), dtype=torch.int32, device=dev)
            out.count_inner = torch.empty(Q, dtype=torch.int32, device=dev)
        if keep_scores:
            out.scores = torch.empty((Q, max(max_valid, 1)), dtype=torch.float32, device=dev)
    _check_topk_out(out, Q, k, k_inner, max_valid, dev)
    ld = int(out.scores.shape[1]) if out.scores is not None else 0
    op = LI_OP_SCORE_TOPK_EXT_SCORES if out.scores is not None else LI_OP_SCORE_TOPK
    nb = workspace_bytes(op, Q, max_valid, H, cache.r, k, 0)
    ws = _workspace(dev, nb, ws)
    c = cache.desc()
    _check(lib().li_score_topk(ctypes.byref(c), ctypes.byref(qs), _ptr(qbuf), _ptr(w), _ptr(bias), H, k, _ptr(out.idx),
                               _ptr(out.count), k_inner, _ptr(out.idx_inner), _ptr(out.count_inner),
                               _ptr(out.scores), ld, _ptr(ws), ws.numel(), _stream(dev)), "li_score_topk")
    return out


def score_topk_noalloc(cache: LatentCache, seq: torch.Tensor, pos: torch.Tensor, max_valid: int,
                       q_tilde: torch.Tensor, w: torch.Tensor, k: int, out: TopK, k_inner: int = 0,
                       bias: Optional[torch.Tensor] = None) -> TopK:
    """li_score_topk_noalloc: li_score_topk on the library's per-GPU scratch
    instead of a workspace.  `out` is required (the call allocates nothing);
    out.scores, when set, receives the scores."""
    dev = cache.device
    qs = _queries(cache, seq, pos, max_valid)
    Q = qs.Q
    H, qbuf = _query_operand(cache, q_tilde, Q)
    _need(w, "w", torch.float32, dev, (Q, H))
    if bias is not None:
        _need(bias, "bias", torch.float32, dev, (Q, H))
    _check_topk_out(out, Q, k, k_inner, max_valid, dev)
    ld = int(out.scores.shape[1]) if out.scores is not None else 0
    c = cache.desc()
    _check(lib().li_score_topk_noalloc(ctypes.byref(c), ctypes.byref(qs), _ptr(qbuf), _ptr(w), _ptr(bias), H, k,
                                       _ptr(out.idx), _ptr(out.count), k_inner, _ptr(out.idx_inner),
                                       _ptr(out.count_inner), _ptr(out.scores), ld, _stream(dev)),
           "li_score_topk_noalloc")
    return out


def hs_select(cache: LatentCache, seq: torch.Tensor, pos: torch.Tensor, max_valid: int, cand: torch.Tensor,
              cand_count: torch.Tensor, q_tilde: torch.Tensor, w: torch.Tensor, k: int, keep_scores: bool = False,
              ws: Optional[torch.Tensor] = None, out: Optional[TopK] = None,
              bias: Optional[torch.Tensor] = None) -> TopK:
    """li_hs_select: rescore the anchor's candidates and take this layer's top-k of them."""
    dev = cache.device
    qs = _queries(cache, seq, pos, max_valid)
    Q = qs.Q
    _need(cand, "cand", torch.int32, dev)
    if cand.dim() != 2 or cand.shape[0] != Q:
        raise ValueError("cand must be [Q][M]")
    M = int(cand.shape[1])
    _need(cand_count, "cand_count", torch.int32, dev, (Q,))
    H, qbuf = _query_operand(cache, q_tilde, Q)
    _need(w, "w", torch.float32, dev, (Q, H))
    if bias is not None:
        _need(bias, "bias", torch.float32, dev, (Q, H))
    if out is None:
        out = TopK(torch.empty((Q, k), dtype=torch.int32, device=dev), torch.empty(Q, dtype=torch.int32, device=dev))
        if keep_scores:
            out.scores = torch.empty((Q, M), dtype=torch.float32, device=dev)
    _need(out.idx, "idx", torch.int32, dev, (Q, k))
    _need(out.count, "count", torch.int32, dev, (Q,))
    if out.scores is not None:
        _need(out.scores, "cand_scores", torch.float32, dev, (Q, M))
    nb = workspace_bytes(LI_OP_HS_SELECT, Q, 0, H, cache.r, k, M)
    ws = _workspace(dev, nb, ws)
    c = cache.desc()
    _check(lib().li_hs_select(ctypes.byref(c), ctypes.byref(qs), _ptr(cand), _ptr(cand_count), M, _ptr(qbuf),
                              _ptr(w), _ptr(bias), H, k, _ptr(out.idx), _ptr(out.count), _ptr(out.scores), _ptr(ws),
                              ws.numel(), _stream(dev)), "li_hs_select")
    return out

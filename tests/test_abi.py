"""CPU tests of the C ABI: the library loads, exports what the header declares,
and rejects bad arguments on the host before anything reaches the GPU.

No compute call runs here: every call below fails validation (or is empty)
and returns before any HIP call.
"""
import ctypes
import os
import re

import pytest

from sparse_attention_token_absorb_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "latentindex.h")
FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        from sparse_attention_token_absorb_amd import build
        build.build()
    return B.lib()


def header_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\bLI_API\s+[\w\s\*]+?\b(li_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    syms = header_symbols()
    assert syms == sorted(B.EXPORTED), syms
    for s in syms:
        assert hasattr(L, s), s


def test_only_the_abi_is_exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    text_syms = sorted(l.split()[-1] for l in out.splitlines() if " T " in l)
    assert text_syms == sorted(header_symbols()), text_syms


def test_version_and_status_strings(L):
    assert L.li_abi_version() == 4
    assert L.li_status_str(0) == b"LI_OK"
    assert L.li_status_str(4) == b"LI_ERR_WORKSPACE"
    assert L.li_status_str(99) == b"LI_ERR_UNKNOWN"


def test_phase_records_only_in_the_instrumented_build(L):
    """The product library records no phases: li_phase_records answers
    LI_ERR_UNSUPPORTED for both decode kernels (without touching the GPU) and
    rejects an unknown kernel id."""
    buf = (ctypes.c_uint64 * 8)()
    assert L.li_phase_records(B.LI_PHASE_SCORE_DECODE_BF16, buf, ctypes.sizeof(buf)) == B.LI_ERR_UNSUPPORTED
    assert L.li_phase_records(B.LI_PHASE_SCORE_DECODE_FP8, None, 0) == B.LI_ERR_UNSUPPORTED
    assert L.li_phase_records(7, buf, ctypes.sizeof(buf)) == B.LI_ERR_SHAPE


def test_fused_filter_mode_knob(L):
    """li_fused_filter takes modes 0..2 (host state only, no GPU work) and
    rejects others; the default mode is restored afterwards."""
    for m in (0, 2, 1):
        assert L.li_fused_filter(m) == B.LI_OK
    assert L.li_fused_filter(3) == B.LI_ERR_SHAPE
    assert L.li_fused_filter(-1) == B.LI_ERR_SHAPE


def cache(**kw):
    d = dict(pool=FAKE.value, block_table=FAKE.value, seq_lens=FAKE.value, batch=1, max_pages=4, page_size=64,
             num_pages=4, r=256, dtype=B.LI_BF16, scales=None)
    d.update(kw)
    return B._Cache(**d)


def queries(**kw):
    d = dict(seq=FAKE.value, pos=FAKE.value, Q=1, max_valid=256)
    d.update(kw)
    return B._Queries(**d)


def score_topk(L, c=None, q=None, H=64, k=16, k_inner=0, inner=None, ws_bytes=1 << 30, ws=FAKE, scores=None, ld=0,
               qt=FAKE, w=FAKE, idx=FAKE, cnt=FAKE):
    c = cache() if c is None else c
    q = queries() if q is None else q
    return L.li_score_topk(ctypes.byref(c) if c is not False else None, ctypes.byref(q) if q is not False else None,
                           qt, w, None, H, k, idx, cnt, k_inner, inner, inner, scores, ld, ws, ws_bytes, None)


def test_score_topk_validation(L):
    assert score_topk(L, c=False) == B.LI_ERR_NULL
    assert score_topk(L, q=False) == B.LI_ERR_NULL
    assert score_topk(L, c=cache(pool=None)) == B.LI_ERR_NULL
    assert score_topk(L, c=cache(page_size=32)) == B.LI_ERR_UNSUPPORTED
    assert score_topk(L, c=cache(r=100)) == B.LI_ERR_UNSUPPORTED
    assert score_topk(L, c=cache(dtype=7)) == B.LI_ERR_UNSUPPORTED
    assert score_topk(L, c=cache(batch=0)) == B.LI_ERR_SHAPE
    assert score_topk(L, q=queries(max_valid=4 * 64 + 1)) == B.LI_ERR_SHAPE
    assert score_topk(L, q=queries(Q=-1)) == B.LI_ERR_SHAPE
    assert score_topk(L, q=queries(seq=None)) == B.LI_ERR_NULL
    assert score_topk(L, H=0) == B.LI_ERR_SHAPE
    assert score_topk(L, H=65) == B.LI_ERR_SHAPE
    assert score_topk(L, k=0) == B.LI_ERR_SHAPE
    assert score_topk(L, k=65537) == B.LI_ERR_SHAPE
    assert score_topk(L, k=16, k_inner=17) == B.LI_ERR_SHAPE
    assert score_topk(L, k=16, k_inner=4, inner=None) == B.LI_ERR_NULL
    assert score_topk(L, qt=None) == B.LI_ERR_NULL
    assert score_topk(L, ws_bytes=16) == B.LI_ERR_WORKSPACE
    assert score_topk(L, ws=None) == B.LI_ERR_WORKSPACE
    assert score_topk(L, scores=FAKE, ld=10) == B.LI_ERR_SHAPE
    assert b"ld=10" in L.li_last_error()
    # nothing to do: Q = 0 succeeds without touching any pointer
    assert score_topk(L, q=queries(Q=0, seq=None, pos=None), qt=None, w=None, idx=None, cnt=None) == B.LI_OK
    assert L.li_last_error() == b""


def test_hs_select_validation(L):
    c, q = cache(), queries()

    def call(M=64, k=16, cand=FAKE, ws_bytes=1 << 30, H=64):
        return L.li_hs_select(ctypes.byref(c), ctypes.byref(q), cand, FAKE, M, FAKE, FAKE, None, H, k, FAKE, FAKE,
                              None, FAKE, ws_bytes, None)

    assert call(M=0) == B.LI_ERR_SHAPE
    assert call(M=70000) == B.LI_ERR_SHAPE
    assert call(k=0) == B.LI_ERR_SHAPE
    assert call(H=100) == B.LI_ERR_SHAPE
    assert call(cand=None) == B.LI_ERR_NULL
    assert call(ws_bytes=8) == B.LI_ERR_WORKSPACE


def test_absorb_and_append_validation(L):
    a = lambda **kw: L.li_absorb_query(kw.get("q", FAKE), FAKE, FAKE, kw.get("Q", 1), kw.get("H", 64), kw.get("d", 128),
                                      kw.get("r", 256), kw.get("dt", B.LI_BF16), None)
    assert a(d=48) == B.LI_ERR_UNSUPPORTED
    assert a(r=96) == B.LI_ERR_UNSUPPORTED
    assert a(dt=B.LI_FP32, r=300) == B.LI_ERR_UNSUPPORTED
    assert a(H=0) == B.LI_ERR_SHAPE
    assert a(Q=-2) == B.LI_ERR_SHAPE
    assert a(q=None) == B.LI_ERR_NULL
    assert a(Q=0) == B.LI_OK
    # no decoder: only for FP8, and only at d == r
    n = lambda **kw: L.li_absorb_query(FAKE, None, FAKE, 1, 64, kw.get("d", 128), kw.get("r", 128),
                                       kw.get("dt", B.LI_FP8), None)
    assert n(dt=B.LI_BF16) == B.LI_ERR_NULL
    assert n(d=128, r=256) == B.LI_ERR_SHAPE
    c = cache()
    assert L.li_append_latent(ctypes.byref(c), FAKE, FAKE, FAKE, -1, None) == B.LI_ERR_SHAPE
    assert L.li_append_latent(ctypes.byref(c), None, FAKE, FAKE, 3, None) == B.LI_ERR_NULL
    assert L.li_append_latent(ctypes.byref(c), None, None, None, 0, None) == B.LI_OK
    c2 = cache(page_size=16)
    assert L.li_append_latent(ctypes.byref(c2), FAKE, FAKE, FAKE, 3, None) == B.LI_ERR_UNSUPPORTED


def test_workspace_sizes(L):
    ws = lambda *a: B.workspace_bytes(*a)
    assert ws(B.LI_OP_SCORE_TOPK, 4, 131072, 64, 256, 2048, 0) > 4 * 131072 * 4
    assert ws(B.LI_OP_SCORE_TOPK_EXT_SCORES, 4, 131072, 64, 256, 2048, 0) < ws(B.LI_OP_SCORE_TOPK, 4, 131072, 64, 256,
                                                                                2048, 0)
    assert ws(B.LI_OP_HS_SELECT, 4, 0, 64, 256, 2048, 8192) >= 4 * 8192 * 4
    assert ws(B.LI_OP_HS_SELECT, 4, 0, 64, 256, 2048, 0) == 0
    assert ws(B.LI_OP_SCORE_TOPK, -1, 10, 64, 256, 16, 0) == 0
    assert ws(99, 1, 10, 64, 256, 16, 0) == 0
    small, big = ws(B.LI_OP_SCORE_TOPK, 2, 1000, 64, 256, 16, 0), ws(B.LI_OP_SCORE_TOPK, 2, 100000, 64, 256, 16, 0)
    assert big > small


def test_every_workspace_starts_with_the_zeroed_region(L):
    """Every op's workspace holds the region the long-row selection keeps
    zeroed (64 queries x 4112 words, the header's LI_WORKSPACE_ZEROED_BYTES)
    ahead of everything else: the smallest workspace of each op is larger
    than it, and the binding's own workspaces come zero-filled."""
    torch = pytest.importorskip("torch")
    zeroed = 64 * 4112 * 4
    hdr = open(os.path.join(ROOT, "include", "latentindex.h")).read()
    assert "#define LI_WORKSPACE_ZEROED_BYTES (64 * 4112 * 4)" in hdr
    for op, mv, M in ((B.LI_OP_SCORE_TOPK, 1, 0), (B.LI_OP_SCORE_TOPK_EXT_SCORES, 1, 0), (B.LI_OP_HS_SELECT, 0, 1)):
        assert B.workspace_bytes(op, 1, mv, 64, 256, 1, M) > zeroed
    w = B.workspace(1000, "cpu")
    assert w.dtype == torch.uint8 and int(w.numel()) == 1000 and int(w.count_nonzero()) == 0


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError):
        B.absorb_query(torch.zeros(1, 4, 32), torch.zeros(32, 64))


def test_fp8_validation_and_sizes(L):
    c = cache(dtype=B.LI_FP8)  # no scales
    assert L.li_append_latent(ctypes.byref(c), FAKE, FAKE, FAKE, 3, None) == B.LI_ERR_NULL
    c = cache(dtype=B.LI_FP8, scales=FAKE.value, r=64)
    assert L.li_append_latent(ctypes.byref(c), FAKE, FAKE, FAKE, 3, None) == B.LI_ERR_UNSUPPORTED
    c = cache(dtype=B.LI_FP8, scales=FAKE.value, r=256)
    assert L.li_append_latent(ctypes.byref(c), None, None, None, 0, None) == B.LI_OK
    assert score_topk(L, c=c, k=0) == B.LI_ERR_SHAPE
    a = lambda **kw: L.li_absorb_query(FAKE, FAKE, FAKE, kw.get("Q", 1), 64, kw.get("d", 128), kw.get("r", 256),
                                      B.LI_FP8, None)
    assert a(r=64) == B.LI_ERR_UNSUPPORTED
    assert a(d=48) == B.LI_ERR_UNSUPPORTED
    assert a(Q=0) == B.LI_OK
    # codes [Q][H][r], then (256-byte aligned) scales [Q][H][r/128] fp32
    assert L.li_fp8_query_scale_offset(3, 64, 256) == 3 * 64 * 256
    assert L.li_fp8_query_bytes(3, 64, 256) == 3 * 64 * 256 + 3 * 64 * 2 * 4
    assert L.li_fp8_query_scale_offset(1, 3, 128) == 512
    assert L.li_fp8_query_bytes(1, 3, 128) == 512 + 3 * 4
    assert L.li_fp8_query_bytes(1, 64, 64) == 0 and L.li_fp8_query_bytes(1, 0, 256) == 0


def test_rope_entry_points_validation(L):
    c = cache()
    rope = lambda F=32, S=2, base=10000.0: ctypes.byref(B._Rope(F, S, base))
    ap = lambda rp, T=3, rows=FAKE, cc=c: L.li_append_latent_rope(ctypes.byref(cc), rows, FAKE, FAKE, T, rp, None)
    assert ap(None) == B.LI_ERR_NULL
    assert ap(rope(F=0)) == B.LI_ERR_SHAPE
    assert ap(rope(F=65)) == B.LI_ERR_SHAPE
    assert ap(rope(S=0)) == B.LI_ERR_SHAPE
    assert ap(rope(F=64, S=3)) == B.LI_ERR_SHAPE          # 2 S F = 384 > r = 256
    assert ap(rope(base=1.0)) == B.LI_ERR_SHAPE
    assert ap(rope(), rows=None) == B.LI_ERR_NULL
    assert ap(rope(), T=-1) == B.LI_ERR_SHAPE
    assert ap(rope(), T=0, rows=None) == B.LI_OK
    assert ap(rope(), cc=cache(page_size=16)) == B.LI_ERR_UNSUPPORTED
    dec = lambda rp, dt=B.LI_BF16, D=FAKE: L.li_rope_decoder(D, FAKE, rp, 64, 128, FAKE, dt, None)
    assert dec(None) == B.LI_ERR_NULL
    assert dec(rope(F=0)) == B.LI_ERR_SHAPE
    assert dec(rope(), dt=B.LI_FP8) == B.LI_ERR_UNSUPPORTED
    assert dec(rope(), D=None) == B.LI_ERR_NULL
    qb = lambda Q=1, d=128, d_rope=64, dt=B.LI_BF16, q=FAKE: L.li_query_bias(q, FAKE, Q, 64, d, d_rope, FAKE, dt, None)
    assert qb(d_rope=200) == B.LI_ERR_SHAPE
    assert qb(Q=-1) == B.LI_ERR_SHAPE
    assert qb(dt=B.LI_FP8) == B.LI_ERR_UNSUPPORTED
    assert qb(q=None) == B.LI_ERR_NULL
    assert qb(Q=0, q=None) == B.LI_OK

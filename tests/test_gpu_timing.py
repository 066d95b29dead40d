"""GPU: the library's kernel timing (li_timing_enable / li_timing_read).

A scoring class times the kernel itself: its events are bound to the one
scoring kernel of each call, so every interval lies inside the interval of a
pair of stream events recorded around the whole call (scoring plus
selection).  The counts are one launch per call of each scoring class, and
nothing is counted while timing is off.  Inputs are seeded random device
tensors; only timing is checked here (parity lives in the other GPU tests).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from sparse_attention_token_absorb_amd import binding as B

pytestmark = pytest.mark.gpu

CLASSES = (B.LI_KERNEL_SCORE_DECODE, B.LI_KERNEL_SCORE_PREFILL, B.LI_KERNEL_SCORE_GATHER, B.LI_KERNEL_SELECT,
           B.LI_KERNEL_ABSORB, B.LI_KERNEL_APPEND)


def say(msg: str) -> None:
    print(f"[timing] {msg}", flush=True)
    sys.stdout.flush()


def _setup(Bn=4, N=32768, r=256, H=64, seed=11):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(seed)
    pages = N // 64
    pool = torch.randn((Bn * pages, 64, r), generator=g, device=dev).to(torch.bfloat16)
    bt = torch.arange(Bn * pages, dtype=torch.int32, device=dev).reshape(Bn, pages)
    cache = B.LatentCache(pool, bt, torch.full((Bn,), N, dtype=torch.int32, device=dev))
    seq = torch.arange(Bn, dtype=torch.int32, device=dev)
    pos = torch.full((Bn,), N - 1, dtype=torch.int32, device=dev)
    qt = torch.randn((Bn, H, r), generator=g, device=dev).to(torch.bfloat16)
    w = torch.rand((Bn, H), generator=g, device=dev)
    return cache, seq, pos, qt, w


def _drain():
    for c in CLASSES:
        B.timing_read(c)


def _timed_calls(fn, stream, calls):
    """(per-call stream intervals in ms); the library's own events run meanwhile."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    B.timing_enable(True)
    try:
        with torch.cuda.stream(stream):
            for a, b in ev:
                a.record(stream)
                fn()
                b.record(stream)
        torch.cuda.synchronize()
    finally:
        B.timing_enable(False)
    return [a.elapsed_time(b) for a, b in ev]


def test_decode_scoring_is_timed_per_kernel():
    cache, seq, pos, qt, w = _setup()
    N, k = 32768, 2048
    stream = torch.cuda.current_stream()
    run = lambda: B.score_topk(cache, seq, pos, N, qt, w, k)
    run()
    torch.cuda.synchronize()
    _drain()
    calls = 5
    wall = _timed_calls(run, stream, calls)
    score_ms, n_score = B.timing_read(B.LI_KERNEL_SCORE_DECODE)
    sel_ms, n_sel = B.timing_read(B.LI_KERNEL_SELECT)
    say(f"decode B=4 N=32768: score {score_ms / calls * 1e3:.2f} us/launch, selection {sel_ms / calls * 1e3:.2f} us, "
        f"call {np.mean(wall) * 1e3:.2f} us")
    assert n_score == calls
    assert n_sel >= calls
    assert 0 < score_ms < sum(wall)
    assert score_ms + sel_ms <= sum(wall) * 1.001 + 1e-3
    for c in (B.LI_KERNEL_SCORE_PREFILL, B.LI_KERNEL_SCORE_GATHER, B.LI_KERNEL_ABSORB, B.LI_KERNEL_APPEND):
        assert B.timing_read(c) == (0.0, 0)
    # nothing is recorded while timing is off
    run()
    torch.cuda.synchronize()
    assert B.timing_read(B.LI_KERNEL_SCORE_DECODE) == (0.0, 0)


def test_hs_follower_scoring_is_timed_per_kernel():
    cache, seq, pos, qt, w = _setup(seed=12)
    N, k, M = 32768, 2048, 8192
    anchor = B.score_topk(cache, seq, pos, N, qt, w, M, k_inner=k)
    torch.cuda.synchronize()
    qt2 = torch.flip(qt, dims=(1,)).contiguous()
    stream = torch.cuda.current_stream()
    run = lambda: B.hs_select(cache, seq, pos, N, anchor.idx, anchor.count, qt2, w, k)
    run()
    torch.cuda.synchronize()
    _drain()
    calls = 4
    wall = _timed_calls(run, stream, calls)
    g_ms, n_g = B.timing_read(B.LI_KERNEL_SCORE_GATHER)
    s_ms, n_s = B.timing_read(B.LI_KERNEL_SELECT)
    say(f"HS follower B=4 M=8192: gather scoring {g_ms / calls * 1e3:.2f} us/launch, call {np.mean(wall) * 1e3:.2f} us")
    assert n_g == calls and n_s >= calls
    assert 0 < g_ms and g_ms + s_ms <= sum(wall) * 1.001 + 1e-3
    assert B.timing_read(B.LI_KERNEL_SCORE_DECODE) == (0.0, 0)

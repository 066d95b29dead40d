#!/usr/bin/env python3
"""Benchmark of the LatentIndex indexer hot path on one MI355X.

One step = one decode step of one layer group (G = 4) for a batch of 4
sequences at 131072 rows of context, run the three ways the long-context
workload names:
  (b) full LatentIndex: the anchor appends the new latent rows, every layer
      absorbs its decoder into its query, scores all rows, selects top-2048;
  (c) hierarchical selection: the anchor selects its top-8192 candidates
      (with its own top-2048 nested), the 3 followers rescore only those;
  (a) the per-layer baseline indexer: 4 separate [N][128] key caches, each
      scored in full with the un-absorbed query.
Inputs are seeded synthetic data resident in HBM before timing starts.  The
step is captured once as a HIP graph and replayed; `value` is indexer rows
scored per second over the whole step.

Extra fields: per-mode µs/layer, the scoring kernel's HBM roofline (kernel
durations from HIP events the library records around each launch), a
context sweep 8K..128K, chunked prefill scoring (4096 queries x 65536 rows,
one layer) against the bf16 MFMA peak, and the fp64 CPU oracle timed on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "indexer decode us/layer + latent rows scored/s, 8K-128K ctx; % HBM peak"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, TFLOP/s
FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, TFLOP/s


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--context", type=int, default=131072)
    ap.add_argument("--batch", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-workloads", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-rope", action="store_true")
    ap.add_argument("--no-model", action="store_true")
    ap.add_argument("--out", default=None, help="also write the JSON line to this file")
    ap.add_argument("--roofline-only", action="store_true",
                    help="only the roofline kernel's cold launches (a 1 GiB scrub before each), for a rocprofv3 "
                         "kernel trace whose average duration is the line's roofline figure; prints their timing")
    ap.add_argument("--counters", choices=("decode", "prefill", "prefill-fp8"), default=None,
                    help="hardware-counter pass, no JSON line: 'decode' runs a few eager full-LatentIndex layers, "
                         "then a plain 1 GiB copy whose counter readings scale the others to bytes; 'prefill' "
                         "('prefill-fp8') runs a few eager chunked-prefill layers on a bf16 (FP8) cache")
    ap.add_argument("--phases", action="store_true",
                    help="per-wave phase timestamps of the decode scoring kernels (bf16 and FP8, cold and warm "
                         "launches) from the instrumented library variant (python -m "
                         "sparse_attention_token_absorb_amd.build phases); prints one JSON line per case")
    return ap.parse_args()


def phase_summary(rec, np):
    """Per-wave phase records (li_phase_records) -> where one launch's time goes.

    Times are microseconds from the earliest wave start (100 MHz clock).
    'first_tile' is when a wave's first tile of rows has landed in LDS, 'loop_end'
    when its stream is done, 'end' when the wave ends (after the score copy-out
    and the histogram flush).  Each entry is [min, median, max] over waves."""
    r = rec[rec[:, 0] != 0].astype(np.int64)
    if len(r) == 0:
        return {"waves": 0}
    rel = (r[:, :5] - r[:, 0].min()) * 0.01
    out = {"waves": int(len(r)), "span_us": round(float(rel[:, 4].max()), 2)}
    for i, name in enumerate(("start", "first_tile", "loop_end", "after_barrier", "end")):
        out[name] = [round(float(v), 2) for v in (rel[:, i].min(), np.median(rel[:, i]), rel[:, i].max())]
    loop = rel[:, 2] - rel[:, 1]
    out["stream_us_per_wave"] = [round(float(v), 2) for v in (loop.min(), np.median(loop), loop.max())]
    out["startup_us_median"] = round(float(np.median(rel[:, 1] - rel[:, 0])), 2)
    out["tail_us_median"] = round(float(np.median(rel[:, 4] - rel[:, 3])), 2)
    xcc = (r[:, 5] >> 32) & 0xF
    out["stream_us_median_by_xcc"] = {int(x): round(float(np.median(loop[xcc == x])), 2) for x in sorted(set(xcc.tolist()))}
    out["loop_end_us_median_by_xcc"] = {int(x): round(float(np.median(rel[xcc == x, 2])), 2)
                                         for x in sorted(set(xcc.tolist()))}
    return out


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the indexer path here is "
              f"single-GPU and has no multi-GPU mode.", file=sys.stderr, flush=True)
        return 2
    import numpy as np
    import torch

    from sparse_attention_token_absorb_amd import binding as B
    from sparse_attention_token_absorb_amd import synth

    if args.phases:
        from sparse_attention_token_absorb_amd import build as hip_build
        if not os.path.exists(hip_build.LIB_PHASES):
            print(f"{hip_build.LIB_PHASES} is not built: python -m sparse_attention_token_absorb_amd.build phases",
                  file=sys.stderr, flush=True)
            return 2
        B.LIB_PATH = hip_build.LIB_PHASES
    B.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bf = torch.bfloat16

    def i32(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(dev)

    def tdev(x, dt):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dt).to(dev)

    if args.counters in ("prefill", "prefill-fp8"):
        pl = setup_prefill(B, synth, dev, bf, i32, tdev, args.context // 2, fp8=args.counters == "prefill-fp8")
        for _ in range(3):
            pl.layer()
        torch.cuda.synchronize()
        log(f"counter pass done: 3 chunked-prefill layers ({args.counters})")
        return 0

    # ------------------------------------------------------------------
    # Inputs (seeded, synthetic), resident on the GPU
    # ------------------------------------------------------------------
    N, Bn = args.context, args.batch
    log(f"generating inputs B={Bn} N={N}")
    g = synth.long_context_b4(N=N, B=Bn)
    H, d, r, k, M, G = g.H, g.d, g.r, g.k, g.M, g.G

    def make_cache(latent, width):
        pool = torch.zeros((g.num_pages, 64, width), dtype=bf, device=dev)
        c = B.LatentCache(pool, i32(g.block_table), i32(g.lens))
        for b in range(Bn):
            n = int(g.lens[b])
            B.append_latent(c, tdev(latent[b], bf), i32(np.full(n, b)), i32(np.arange(n)))
        return c

    cache = make_cache(g.latent, r)
    key_caches = [make_cache(g.keys_a[l], d) for l in range(G)]
    seq, pos = i32(g.qseq), i32(g.qpos)
    q = [tdev(g.q[l], bf) for l in range(G)]
    W = [tdev(g.W[l], bf) for l in range(G)]
    w = [torch.from_numpy(g.w[l]).to(dev) for l in range(G)]
    new_rows = torch.stack([tdev(g.latent[b][N - 1], bf) for b in range(Bn)]).contiguous()
    new_seq, new_pos = i32(np.arange(Bn)), i32(np.full(Bn, N - 1))
    qt = [torch.empty((Bn, H, r), dtype=bf, device=dev) for _ in range(G)]
    ws = B.workspace(B.workspace_bytes(B.LI_OP_SCORE_TOPK, Bn, N, H, r, M, 0), dev)
    ws_hs = B.workspace(B.workspace_bytes(B.LI_OP_HS_SELECT, Bn, 0, H, r, k, M), dev)

    def topk_out(kk, inner=0):
        o = B.TopK(torch.empty((Bn, kk), dtype=torch.int32, device=dev), torch.empty(Bn, dtype=torch.int32, device=dev))
        if inner:
            o.idx_inner = torch.empty((Bn, inner), dtype=torch.int32, device=dev)
            o.count_inner = torch.empty(Bn, dtype=torch.int32, device=dev)
        return o

    out_b = [topk_out(k) for _ in range(G)]
    out_anchor = topk_out(M, k)
    out_f = [topk_out(k) for _ in range(G - 1)]
    out_a = [topk_out(k) for _ in range(G)]
    del g.keys_a

    def prep():
        B.append_latent(cache, new_rows, new_seq, new_pos)
        for l in range(G):
            B.absorb_query(q[l], W[l], out=qt[l])

    def mode_b(max_valid=N, sq=None, sp=None):
        for l in range(G):
            B.score_topk(cache, sq if sq is not None else seq, sp if sp is not None else pos, max_valid, qt[l], w[l], k,
                         ws=ws, out=out_b[l])

    def mode_c():
        B.score_topk(cache, seq, pos, N, qt[0], w[0], M, k_inner=k, ws=ws, out=out_anchor)
        for l in range(1, G):
            B.hs_select(cache, seq, pos, N, out_anchor.idx, out_anchor.count, qt[l], w[l], k, ws=ws_hs, out=out_f[l - 1])

    def mode_a():
        for l in range(G):
            B.score_topk(key_caches[l], seq, pos, N, q[l], w[l], k, ws=ws, out=out_a[l])

    def step():
        prep()
        mode_b()
        mode_c()
        mode_a()

    stream = torch.cuda.Stream(device=dev)

    if args.counters == "decode":
        B.fused_filter(B.FUSED_FILTER_OFF)  # the scoring stream alone, as the roofline times it
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            mode_b()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"counter pass done: 3 x {G} full-LatentIndex layers, 3 x copy of {src.numel() * 4} bytes")
        return 0

    if args.roofline_only:
        B.fused_filter(B.FUSED_FILTER_OFF)  # the scoring stream alone (the filter pass in its own kernel)
        scrub = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        sink = torch.empty(1, dtype=torch.float32, device=dev)
        bytes_launch = Bn * N * 2 * r + Bn * (H * r * 2 + H * 4)
        with torch.cuda.stream(stream):
            B.score_topk(cache, seq, pos, N, qt[0], w[0], k, ws=ws, out=out_b[0])  # first launch, untimed
        torch.cuda.synchronize()
        B.timing_read(B.LI_KERNEL_SCORE_DECODE)
        B.timing_enable(True)
        with torch.cuda.stream(stream):
            for _ in range(args.steps):
                for l in range(G):
                    torch.sum(scrub, dim=0, keepdim=True, out=sink)
                    B.absorb_query(q[l], W[l], out=qt[l])
                    B.score_topk(cache, seq, pos, N, qt[l], w[l], k, ws=ws, out=out_b[l])
        torch.cuda.synchronize()
        B.timing_enable(False)
        tot, n = B.timing_read(B.LI_KERNEL_SCORE_DECODE)
        us = tot / max(n, 1) * 1e3
        print(json.dumps({"kernel": "k_score_decode (r=256, 64 heads, B=4, N=131072, cold)", "launches": n,
                          "avg_launch_us": round(us, 2), "bytes_per_launch": bytes_launch,
                          "achieved_GBs": round(bytes_launch / us / 1e3, 1)}), flush=True)
        return 0

    if args.phases:
        # the same launches as the roofline's (cold: a 1 GiB read-only scrub
        # before each; warm: back to back), bf16 and FP8 caches of the latent
        scrub = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        sink = torch.empty(1, dtype=torch.float32, device=dev)
        f8pool = torch.zeros((g.num_pages, 64, r), dtype=torch.uint8, device=dev)
        f8sc = torch.zeros((g.num_pages, 64, r // 128), dtype=torch.float32, device=dev)
        f8cache = B.LatentCache(f8pool, i32(g.block_table), i32(g.lens), f8sc)
        for b in range(Bn):
            B.append_latent(f8cache, tdev(g.latent[b], bf), i32(np.full(N, b)), i32(np.arange(N)))
        for l in range(G):
            B.absorb_query(q[l], W[l], out=qt[l])
        f8q = B.absorb_query(q[0], W[0], fp8=True)
        cases = (("bf16", B.LI_PHASE_SCORE_DECODE_BF16, lambda: B.score_topk(cache, seq, pos, N, qt[0], w[0], k, ws=ws,
                                                                               out=out_b[0])),
                 ("fp8", B.LI_PHASE_SCORE_DECODE_FP8, lambda: B.score_topk(f8cache, seq, pos, N, f8q, w[0], k, ws=ws,
                                                                             out=out_b[0])))
        for name, which, run in cases:
            for _ in range(3):
                run()
            for rep in range(args.steps):
                for cold in (True, False):
                    B.phase_clear(which)
                    if cold:
                        torch.sum(scrub, dim=0, keepdim=True, out=sink)
                    torch.cuda.synchronize()
                    B.timing_read(B.LI_KERNEL_SCORE_DECODE)
                    B.timing_enable(True)
                    run()
                    torch.cuda.synchronize()
                    B.timing_enable(False)
                    ms, n = B.timing_read(B.LI_KERNEL_SCORE_DECODE)
                    summary = phase_summary(B.phase_records(which), np)
                    summary = {"kernel": f"{name} decode scoring, B={Bn}, N={N}", "launch": "cold" if cold else "warm",
                               "rep": rep, "event_us": round(ms / max(n, 1) * 1e3, 2), **summary}
                    print(json.dumps(summary), flush=True)
        return 0

    def capture(fn):
        with torch.cuda.stream(stream):
            fn()  # eager warm-up on the capture stream
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            fn()
        torch.cuda.synchronize()
        return graph

    def time_graph(graph, reps, warm=2):
        for _ in range(warm):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / reps

    # ------------------------------------------------------------------
    # Headline: the whole step as one graph
    # ------------------------------------------------------------------
    log("capturing the step")
    g_step = capture(step)
    for _ in range(args.warmup):
        g_step.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g_step.replay()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    rows_b = G * Bn * N
    rows_c = Bn * N + (G - 1) * Bn * min(M, N)
    rows_a = G * Bn * N
    rows_step = rows_b + rows_c + rows_a
    value = rows_step / (ms_per_step * 1e-3)
    log(f"step {ms_per_step:.3f} ms, {value / 1e9:.2f} G rows/s")

    # graph replays must agree with eager execution
    snap = [o.idx.clone() for o in out_b] + [out_anchor.idx.clone()] + [o.idx.clone() for o in out_f]
    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    for a, bb in zip(snap, [o.idx for o in out_b] + [out_anchor.idx] + [o.idx for o in out_f]):
        for i in range(Bn):
            sa, sb = set(a[i].tolist()), set(bb[i].tolist())
            assert len(sa ^ sb) <= 2, "graph replay disagrees with eager execution"

    # ------------------------------------------------------------------
    # Per-mode µs/layer (graphs of one mode each)
    # ------------------------------------------------------------------
    reps = max(args.steps, 10)
    ms_prep = time_graph(capture(prep), reps)
    ms_b = time_graph(capture(mode_b), reps)
    ms_c = time_graph(capture(mode_c), reps)
    ms_a = time_graph(capture(mode_a), reps)
    modes = {
        "append_plus_absorb_x4_us": round(ms_prep * 1e3, 2),
        "full_latentindex_us_per_layer": round(ms_b * 1e3 / G, 2),
        "hs_us_per_group": round(ms_c * 1e3, 2),
        "hs_us_per_layer_avg": round(ms_c * 1e3 / G, 2),
        "baseline_per_layer_indexer_us_per_layer": round(ms_a * 1e3 / G, 2),
        "group_us": {"full": round(ms_b * 1e3, 1), "hs": round(ms_c * 1e3, 1), "baseline": round(ms_a * 1e3, 1)},
        "rows_per_step": {"full": rows_b, "hs": rows_c, "baseline": rows_a},
        "hs_speedup_over_baseline_group": round(ms_a / ms_c, 3) if ms_c > 0 else None,
    }
    log(f"modes {modes}")

    # ------------------------------------------------------------------
    # Roofline of the decode scoring kernel (HIP events bound to each launch's
    # kernel start and end on its launch stream)
    # ------------------------------------------------------------------
    def kernel_time(fn, cls, reps_, fused=False):
        # Kernel-level timing.  By default the long-row selection's filter
        # pass runs in a kernel of its own here, so a scoring launch is the
        # latent stream alone (its roofline); fused=True times the launch as
        # the decode step runs it, with the filter pass inside.
        B.timing_read(cls)
        B.timing_enable(True)
        B.fused_filter(B.FUSED_FILTER_ON if fused else B.FUSED_FILTER_OFF)
        try:
            with torch.cuda.stream(stream):
                for _ in range(reps_):
                    fn()
            torch.cuda.synchronize()
        finally:
            B.timing_enable(False)
            B.fused_filter(B.FUSED_FILTER_ON)
        tot, n = B.timing_read(cls)
        for other in range(6):  # recycle the events of the other classes
            if other != cls:
                B.timing_read(other)
        return tot / max(n, 1), n

    bytes_row = 2 * r
    bytes_query = H * r * 2 + H * 4
    bytes_launch = Bn * N * bytes_row + Bn * bytes_query
    score_ms, n_launch = kernel_time(mode_b, B.LI_KERNEL_SCORE_DECODE, reps)
    sel_ms, _ = kernel_time(mode_b, B.LI_KERNEL_SELECT, reps)
    fused_ms, _ = kernel_time(mode_b, B.LI_KERNEL_SCORE_DECODE, reps, fused=True)
    fused_sel_ms, _ = kernel_time(mode_b, B.LI_KERNEL_SELECT, reps, fused=True)
    achieved = bytes_launch / (score_ms * 1e-3) / 1e9
    # cold (the roofline figure): reading 1 GiB of other data between
    # launches evicts the 256 MB Infinity Cache (a read-only scrub leaves no
    # dirty lines to write back)
    scrub = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.empty(1, dtype=torch.float32, device=dev)

    def cold_b():
        # each layer as a decode step runs it: absorption, then scoring, with
        # the latent evicted from every cache in between layers
        for l in range(G):
            torch.sum(scrub, dim=0, keepdim=True, out=sink)
            B.absorb_query(q[l], W[l], out=qt[l])
            B.score_topk(cache, seq, pos, N, qt[l], w[l], k, ws=ws, out=out_b[l])

    cold_ms, n_cold = kernel_time(cold_b, B.LI_KERNEL_SCORE_DECODE, max(reps // 2, 4))
    del scrub
    # The 268 MB latent is about the size of the 256 MB last-level cache, so
    # warm repeats are partly served from it; the same kernel over pools of
    # 2x and 4x that size (8 and 16 sequences of N rows, random contents)
    # streams from HBM only.
    large = {}
    for nb in (2 * Bn, 4 * Bn):
        pool_l = torch.randn((nb * (N // 64), 64, r), device=dev).to(bf)
        cache_l = B.LatentCache(pool_l, i32(np.arange(nb * (N // 64), dtype=np.int32).reshape(nb, N // 64)),
                                i32([N] * nb))
        qt_l = torch.randn((nb, H, r), device=dev).to(bf)
        w_l = torch.rand((nb, H), device=dev)
        seq_l, pos_l = i32(np.arange(nb)), i32([N - 1] * nb)
        ws_l = B.workspace(B.workspace_bytes(B.LI_OP_SCORE_TOPK, nb, N, H, r, k, 0), dev)
        out_l = B.TopK(torch.empty((nb, k), dtype=torch.int32, device=dev), torch.empty(nb, dtype=torch.int32, device=dev))
        run_l = lambda: B.score_topk(cache_l, seq_l, pos_l, N, qt_l, w_l, k, ws=ws_l, out=out_l)
        with torch.cuda.stream(stream):  # the timed launches' stream: warm-ups must not overlap them
            for _ in range(2):
                run_l()
        l_ms, _ = kernel_time(run_l, B.LI_KERNEL_SCORE_DECODE, max(reps // 2, 4))
        l_bytes = nb * N * bytes_row + nb * bytes_query
        large[f"B{nb}"] = {"bytes_per_launch": l_bytes, "avg_launch_us": round(l_ms * 1e3, 2),
                           "achieved_GBs": round(l_bytes / (l_ms * 1e-3) / 1e9, 1)}
        del pool_l, cache_l, ws_l
    torch.cuda.empty_cache()
    a_score_ms, _ = kernel_time(mode_a, B.LI_KERNEL_SCORE_DECODE, reps)
    a_bytes = Bn * N * 2 * d + Bn * (H * d * 2 + H * 4)
    f_ms, _ = kernel_time(mode_c, B.LI_KERNEL_SCORE_GATHER, reps)
    f_bytes = Bn * min(M, N) * (bytes_row + 4) + Bn * bytes_query
    cold_gbs = bytes_launch / (cold_ms * 1e-3) / 1e9
    roofline = {
        "bound": "hbm", "achieved": round(cold_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(cold_gbs / HBM_PEAK_GBS, 4),
        "traffic": measured_traffic(os.path.join(ROOT, "profiles", "score_decode_r256_h64_b4_n131072.md"),
                                    os.path.join(ROOT, "sparse_attention_token_absorb_amd", "csrc", "score.hip")),
        "kernel": f"k_score_decode<r={r},64 heads> (full LatentIndex, B={Bn}, N={N})",
        "timing": "cold: a 1 GiB read-only scrub before every launch evicts the 256 MB last-level cache; "
                  "HIP events bound to the kernel's own start and end on its launch stream",
        "avg_launch_us": round(cold_ms * 1e3, 2), "launches": n_cold, "bytes_per_launch": bytes_launch,
        "warm_avg_launch_us": round(score_ms * 1e3, 2), "warm_launches": n_launch,
        "warm_achieved_GBs": round(achieved, 1), "warm_frac": round(achieved / HBM_PEAK_GBS, 4),
        "beyond_llc": large,
        "with_fused_filter": {"score_plus_filter_us": round(fused_ms * 1e3, 2),
                              "select_after_us": round(fused_sel_ms * 1e3, 2),
                              "note": "the decode step's form: the selection's filter pass runs in the scoring "
                                      "launch, the final kernel after it; the figures above time the scoring "
                                      "stream alone"},
        "separate_filter_select_us": round(sel_ms * 1e3, 2),
        "baseline_r128_score_us": round(a_score_ms * 1e3, 2),
        "baseline_r128_GBs": round(a_bytes / (a_score_ms * 1e-3) / 1e9, 1),
        "hs_follower_gather_score_us": round(f_ms * 1e3, 2),
        "hs_follower_gather_GBs": round(f_bytes / (f_ms * 1e-3) / 1e9, 1),
    }
    log(f"roofline {roofline}")

    # ------------------------------------------------------------------
    # Context sweep 8K..128K (full LatentIndex, same cache, shorter prefixes)
    # ------------------------------------------------------------------
    sweep = {}
    if not args.no_sweep:
        for n_ctx in (8192, 16384, 32768, 65536, 131072):
            if n_ctx > N:
                continue
            sp = i32(np.full(Bn, n_ctx - 1))
            gr = capture(lambda: mode_b(n_ctx, seq, sp))
            ms = time_graph(gr, reps)
            sc_ms, _ = kernel_time(lambda: mode_b(n_ctx, seq, sp), B.LI_KERNEL_SCORE_DECODE, reps)
            by = Bn * n_ctx * bytes_row + Bn * bytes_query
            sweep[str(n_ctx)] = {"us_per_layer": round(ms * 1e3 / G, 2),
                                 "rows_per_s": round(G * Bn * n_ctx / (ms * 1e-3), 1),
                                 "score_kernel_us": round(sc_ms * 1e3, 2),
                                 "score_frac_hbm": round(by / (sc_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            del gr
        log(f"sweep {sweep}")

    # ------------------------------------------------------------------
    # The two other decode workloads: a single 8K sequence (full
    # LatentIndex on all four layers) and 16 ragged paged sequences of
    # 16K-32K rows (full LatentIndex and HS); each layer absorbs
    # its decoder, scores and selects, as one captured graph per mode
    # ------------------------------------------------------------------
    workloads = {}
    if not args.no_workloads:
        for cname, gc in (("decode_b1_n8192", synth.decode_b1_n8192()), ("ragged_paged_b16_n16k_32k", synth.ragged_paged_b16())):
            log(f"{cname} inputs")
            Bc = gc.B
            pool_c = torch.zeros((gc.num_pages, 64, gc.r), dtype=bf, device=dev)
            cache_c = B.LatentCache(pool_c, i32(gc.block_table), i32(gc.lens))
            for b in range(Bc):
                n_b = int(gc.lens[b])
                B.append_latent(cache_c, tdev(gc.latent[b][:n_b], bf), i32(np.full(n_b, b)), i32(np.arange(n_b)))
            seq_c, pos_c = i32(gc.qseq), i32(gc.qpos)
            n_q = [int(min(gc.qpos[i] + 1, gc.lens[gc.qseq[i]])) for i in range(gc.Q)]
            Nc = max(n_q)
            q_c = [tdev(gc.q[l], bf) for l in range(gc.G)]
            W_c = [tdev(gc.W[l], bf) for l in range(gc.G)]
            w_c = [torch.from_numpy(gc.w[l]).to(dev) for l in range(gc.G)]
            qt_c = [torch.empty((gc.Q, gc.H, gc.r), dtype=bf, device=dev) for _ in range(gc.G)]
            ws_c = B.workspace(B.workspace_bytes(B.LI_OP_SCORE_TOPK, gc.Q, Nc, gc.H, gc.r, gc.M, 0), dev)
            ws_hc = B.workspace(B.workspace_bytes(B.LI_OP_HS_SELECT, gc.Q, 0, gc.H, gc.r, gc.k, gc.M), dev)
            ti = lambda *shape: torch.empty(shape, dtype=torch.int32, device=dev)
            o_full = [B.TopK(ti(gc.Q, gc.k), ti(gc.Q)) for _ in range(gc.G)]
            o_anc = B.TopK(ti(gc.Q, gc.M), ti(gc.Q), ti(gc.Q, gc.k), ti(gc.Q))

            def full_c():
                for l in range(gc.G):
                    B.absorb_query(q_c[l], W_c[l], out=qt_c[l])
                    B.score_topk(cache_c, seq_c, pos_c, Nc, qt_c[l], w_c[l], gc.k, ws=ws_c, out=o_full[l])

            def hs_c():
                for l in range(gc.G):
                    B.absorb_query(q_c[l], W_c[l], out=qt_c[l])
                    if l == 0:
                        B.score_topk(cache_c, seq_c, pos_c, Nc, qt_c[0], w_c[0], gc.M, k_inner=gc.k, ws=ws_c,
                                     out=o_anc)
                    else:
                        B.hs_select(cache_c, seq_c, pos_c, Nc, o_anc.idx, o_anc.count, qt_c[l], w_c[l], gc.k, ws=ws_hc,
                                    out=o_full[l])

            entry = {"batch": Bc, "rows_per_query": [min(n_q), max(n_q)]}
            gr = capture(full_c)
            ms_f = time_graph(gr, reps)
            del gr
            entry["full_latentindex_us_per_layer"] = round(ms_f * 1e3 / gc.G, 2)
            entry["full_rows_per_s"] = round(gc.G * sum(n_q) / (ms_f * 1e-3), 1)
            if Bc > 1:
                gr = capture(hs_c)
                ms_h = time_graph(gr, reps)
                del gr
                entry["hs_us_per_group"] = round(ms_h * 1e3, 2)
                entry["hs_rows_per_s"] = round((sum(n_q) + (gc.G - 1) * sum(min(gc.M, n) for n in n_q)) /
                                               (ms_h * 1e-3), 1)
                entry["hs_speedup_over_full_group"] = round(ms_f / ms_h, 3)
            workloads[cname] = entry
            del cache_c, pool_c, ws_c, ws_hc, gc
            torch.cuda.empty_cache()
        log(f"workloads {workloads}")

    # ------------------------------------------------------------------
    # Segmented FP8 cache (same latent, rotated and quantized on append):
    # full LatentIndex x4 layers and HS, decode scoring against HBM
    # ------------------------------------------------------------------
    fp8 = None
    if not args.no_fp8:
        f8pool = torch.zeros((g.num_pages, 64, r), dtype=torch.uint8, device=dev)
        f8sc = torch.zeros((g.num_pages, 64, r // 128), dtype=torch.float32, device=dev)
        f8cache = B.LatentCache(f8pool, i32(g.block_table), i32(g.lens), f8sc)
        for b in range(Bn):
            B.append_latent(f8cache, tdev(g.latent[b], bf), i32(np.full(N, b)), i32(np.arange(N)))
        f8q = [B.absorb_query(q[l], W[l], fp8=True) for l in range(G)]

        def f8_prep():
            B.append_latent(f8cache, new_rows, new_seq, new_pos)
            for l in range(G):
                B.absorb_query(q[l], W[l], out=f8q[l], fp8=True)

        def f8_full():
            for l in range(G):
                B.score_topk(f8cache, seq, pos, N, f8q[l], w[l], k, ws=ws, out=out_b[l])

        def f8_hs():
            B.score_topk(f8cache, seq, pos, N, f8q[0], w[0], M, k_inner=k, ws=ws, out=out_anchor)
            for l in range(1, G):
                B.hs_select(f8cache, seq, pos, N, out_anchor.idx, out_anchor.count, f8q[l], w[l], k, ws=ws_hs,
                            out=out_f[l - 1])

        f8_ms_prep = time_graph(capture(f8_prep), reps)
        f8_ms_full = time_graph(capture(f8_full), reps)
        f8_ms_hs = time_graph(capture(f8_hs), reps)
        f8_score_ms, _ = kernel_time(f8_full, B.LI_KERNEL_SCORE_DECODE, reps)
        scrub8 = torch.ones(1 << 28, dtype=torch.float32, device=dev)

        def f8_cold():
            for l in range(G):
                torch.sum(scrub8, dim=0, keepdim=True, out=sink)
                B.absorb_query(q[l], W[l], out=f8q[l], fp8=True)
                B.score_topk(f8cache, seq, pos, N, f8q[l], w[l], k, ws=ws, out=out_b[l])

        f8_cold_ms, _ = kernel_time(f8_cold, B.LI_KERNEL_SCORE_DECODE, max(reps // 2, 4))
        del scrub8
        f8_bytes_row = r + (r // 128) * 4
        f8_bytes = Bn * N * f8_bytes_row + Bn * (H * r + H * (r // 128) * 4 + H * 4)
        f8_gbs = f8_bytes / (f8_score_ms * 1e-3) / 1e9
        fp8 = {"append_plus_absorb_x4_us": round(f8_ms_prep * 1e3, 2),
               "full_latentindex_us_per_layer": round(f8_ms_full * 1e3 / G, 2),
               "hs_us_per_group": round(f8_ms_hs * 1e3, 2),
               "score_kernel_us": round(f8_score_ms * 1e3, 2), "bytes_per_launch": f8_bytes,
               "score_GBs": round(f8_gbs, 1), "score_frac_hbm": round(f8_gbs / HBM_PEAK_GBS, 4),
               "cold_score_kernel_us": round(f8_cold_ms * 1e3, 2),
               "cold_score_frac_hbm": round(f8_bytes / (f8_cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               "rows_per_s_full": round(G * Bn * N / (f8_ms_full * 1e-3), 1)}
        log(f"fp8 {fp8}")
        del f8pool, f8sc, f8cache, f8q

    # ------------------------------------------------------------------
    # RoPE-compatible structured decoder (32 rotary frequencies x 2 sources
    # + 128 NoPE columns of the same 256-wide latent, 64 + 64 wide native
    # keys): rotated append + lowered-decoder absorption + bias per layer,
    # then full LatentIndex with the bias in the scoring epilogue
    # ------------------------------------------------------------------
    rope = None
    if not args.no_rope:
        F_, S_ = 32, 2
        rg = synth.make_rope(11, G=G, F=F_, S=S_, d_nope=d - 2 * F_, r_nope=r - 2 * S_ * F_)
        Wd = [B.rope_decoder(tdev(rg.D[l], bf), tdev(rg.Wn[l], bf), (F_, S_)) for l in range(G)]
        betas = [torch.from_numpy(rg.beta[l]).to(dev) for l in range(G)]
        qt_r = [B.absorb_query(q[l], Wd[l]) for l in range(G)]
        bias_r = [B.query_bias(q[l], betas[l], 2 * F_) for l in range(G)]

        def r_prep():
            B.append_latent_rope(cache, new_rows, new_seq, new_pos, (F_, S_))
            for l in range(G):
                B.absorb_query(q[l], Wd[l], out=qt_r[l])
                B.query_bias(q[l], betas[l], 2 * F_, out=bias_r[l])

        def r_full():
            for l in range(G):
                B.score_topk(cache, seq, pos, N, qt_r[l], w[l], k, ws=ws, out=out_b[l], bias=bias_r[l])

        r_ms_prep = time_graph(capture(r_prep), reps)
        r_ms_full = time_graph(capture(r_full), reps)
        r_score_ms, _ = kernel_time(r_full, B.LI_KERNEL_SCORE_DECODE, reps)
        rope = {"layout": f"{F_} frequencies x {S_} sources rotary + {r - 2 * S_ * F_} NoPE of r={r}; native key "
                          f"{2 * F_} rotary + {d - 2 * F_} NoPE",
                "append_rope_plus_absorb_plus_bias_x4_us": round(r_ms_prep * 1e3, 2),
                "full_latentindex_with_bias_us_per_layer": round(r_ms_full * 1e3 / G, 2),
                "score_kernel_with_bias_us": round(r_score_ms * 1e3, 2),
                "score_frac_hbm_with_bias": round(bytes_launch / (r_score_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"rope {rope}")

    # ------------------------------------------------------------------
    # Whole-model indexer step: a 61-layer DeepSeek-V3.2-shaped layer map
    # ------------------------------------------------------------------
    model = None
    if not args.no_model:
        model = model_step(B, dev, i32, capture, time_graph, reps)
        log(f"model {model}")

    # ------------------------------------------------------------------
    # CPU baseline: the fp64 oracle on a bounded sample of the same workload
    # ------------------------------------------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        # the group's layers in turn until about 10 s of CPU work is done
        t0 = time.perf_counter()
        rows_done = 0
        layers_done = 0
        while layers_done < 256:
            l = layers_done % G
            oracle.full_layer(g.q[l], g.W[l], g.w[l], g.latent, g.qseq, g.qpos, g.lens, k)
            rows_done += Bn * N
            layers_done += 1
            if time.perf_counter() - t0 > 10.0:
                break
        el = time.perf_counter() - t0
        cpu = {"value": round(rows_done / el, 1), "unit": "rows/s", "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"full LatentIndex (mode b) at B={Bn}, N={N}: {layers_done} layer passes (the group's "
                         f"{G} layers in turn) x {Bn} queries x {N} rows, each absorb + fp64 scoring + top-{k} "
                         f"sort; {el:.1f} s on {cpu_model()}"}
        if not args.no_prefill:
            # the chunked-prefill layer: 64 evenly spaced query rows (first and
            # last included), each absorb + fp64 scoring of its causal prefix +
            # top-k; extrapolated to the chunk's 4096 rows
            pf = synth.make_prefill("prefill", 5, N=N // 2, Qn=4096, r=256, H=H, d=d, G=1, k=k)
            rows = sorted(set(np.linspace(0, pf.Q - 1, 64).round().astype(int).tolist()))
            t0 = time.perf_counter()
            oracle.full_layer(pf.q[0], pf.W[0], pf.w[0], pf.latent, pf.qseq, pf.qpos, pf.lens, pf.k, rows)
            el_p = time.perf_counter() - t0
            pairs_s = sum(min(int(pf.qpos[i]) + 1, int(pf.lens[0])) for i in rows)
            pairs_all = sum(min(int(p_) + 1, int(pf.lens[0])) for p_ in pf.qpos)
            cpu["prefill"] = {"value": round(pairs_s / el_p, 1), "unit": "query-row pairs scored/s",
                              "extrapolated_ms_per_layer": round(el_p * pairs_all / pairs_s * 1e3, 1),
                              "extrapolated": True, "cores": oracle.num_threads(), "kind": "oracle",
                              "sample": f"{len(rows)} of {pf.Q} query rows (evenly spaced, first and last included) "
                                        f"of one chunked-prefill layer ({pf.Q} queries at positions "
                                        f"{int(pf.qpos[0])}..{int(pf.qpos[-1])} of a {int(pf.lens[0])}-row cache): "
                                        f"{el_p:.1f} s; the layer time is that x {pairs_all}/{pairs_s} valid pairs"}
            del pf
        log(f"cpu baseline {cpu}")

    # ------------------------------------------------------------------
    # Chunked prefill scoring: 4096 queries x 65536 causal rows, one layer
    # ------------------------------------------------------------------
    prefill = None
    if not args.no_prefill:
        del cache, key_caches
        torch.cuda.empty_cache()
        log("prefill inputs")
        pl = setup_prefill(B, synth, dev, bf, i32, tdev, N // 2)
        with torch.cuda.stream(stream):
            pl.layer()
        torch.cuda.synchronize()
        preps = 5
        sc_ms, _ = kernel_time(pl.layer, B.LI_KERNEL_SCORE_PREFILL, preps)
        sel_ms, _ = kernel_time(pl.layer, B.LI_KERNEL_SELECT, preps)
        ab_ms, _ = kernel_time(pl.layer, B.LI_KERNEL_ABSORB, preps)
        flops = 2.0 * H * r * pl.pairs
        tf = flops / (sc_ms * 1e-3) / 1e12
        prefill = {"workload": f"{pl.Q} queries at positions {pl.n - pl.Q}..{pl.n - 1} of a {pl.n}-row cache, "
                               f"one layer",
                   "score_ms": round(sc_ms, 3), "tflops": round(tf, 1), "peak_tflops": BF16_PEAK_TFLOPS,
                   "frac_mfma": round(tf / BF16_PEAK_TFLOPS, 4), "select_ms": round(sel_ms, 3),
                   "absorb_ms": round(ab_ms, 3), "valid_pairs": pl.pairs}
        if not args.no_rope:
            pl.bias = torch.randn((pl.Q, H), dtype=torch.float32, device=dev)
            b_ms, _ = kernel_time(pl.layer, B.LI_KERNEL_SCORE_PREFILL, preps)
            prefill["score_ms_with_bias"] = round(b_ms, 3)
            pl.bias = None
        log(f"prefill {prefill}")
        if not args.no_fp8:
            del pl
            torch.cuda.empty_cache()
            pf = setup_prefill(B, synth, dev, bf, i32, tdev, N // 2, fp8=True)
            with torch.cuda.stream(stream):
                pf.layer()
            torch.cuda.synchronize()
            f_sc, _ = kernel_time(pf.layer, B.LI_KERNEL_SCORE_PREFILL, preps)
            f_sel, _ = kernel_time(pf.layer, B.LI_KERNEL_SELECT, preps)
            f_ab, _ = kernel_time(pf.layer, B.LI_KERNEL_ABSORB, preps)
            f_tf = flops / (f_sc * 1e-3) / 1e12
            prefill["fp8"] = {"score_ms": round(f_sc, 3), "tflops": round(f_tf, 1), "peak_tflops": FP8_PEAK_TFLOPS,
                              "frac_mfma": round(f_tf / FP8_PEAK_TFLOPS, 4), "select_ms": round(f_sel, 3),
                              "absorb_ms": round(f_ab, 3)}
            log(f"prefill fp8 {prefill['fp8']}")

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"decode step of one layer group, B={Bn}, context {N}: full LatentIndex x{G} layers "
                               f"+ HS (M={M}) + per-layer baseline indexer x{G}",
                   "batch": Bn, "context": N, "heads": H, "d": d, "r": r, "k": k, "M": M, "group": G,
                   "parallelism": "single GPU"},
        "modes": modes, "roofline": roofline, "sweep": sweep, "workloads": workloads, "fp8": fp8, "rope": rope,
        "model": model,
        "prefill": prefill, "cpu_baseline": cpu, "device": device_facts(dev),
    }
    s = json.dumps(line)
    print(s, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(s + "\n")
    return 0


def model_step(B, dev, i32, capture, time_graph, reps):
    """Indexer work of one decode step (batch 1) over a 61-layer map shaped
    like the pages' DeepSeek-V3.2 setting (§C.3, §C.4, §B.3): layer 0 keeps
    its own indexer, layers 1-60 form 15 groups of G = 4 (and, as the pages'
    G = 8 variant of §4.4 and §A.5, 7 groups of 8 plus one of 4).  Every cache
    is segmented FP8 as in the pages' inference (§B.2, §C.1): native per-layer
    keys 128 wide (128 code bytes + one scale: the 132 B per token and layer
    of §B.1), group latents 256 wide.  The step is the package's
    IndexerModel.step (append, query absorption or quantization, scoring and
    selection for every layer) under each method:
      dsa         every layer scores its own keys over the whole prefix
      latentindex layer 0 as dsa; each group caches one latent, every layer
                  scores it with its absorbed query and selects top-2048
      hs          as latentindex, but the anchor proposes its top-8192 and the
                  group's followers rescore only those (§3.2, §C.4)
      indexcache  layer 0 and every group's anchor as dsa; followers reuse
                  the anchor's selection (no work)
    Inputs are seeded device-side normals; only timing is reported."""
    import numpy as np
    import torch
    from sparse_attention_token_absorb_amd.model import IndexerModel, LayerMap
    L_max, H, d, r, k, M = 131072, 64, 128, 256, 2048, 8192
    maps = {"G4": LayerMap.grouped(61, 4), "G8": LayerMap.grouped(61, 8)}
    n_layers = 61
    n_groups = max(len(m.groups) for m in maps.values())
    bf = torch.bfloat16
    gen = torch.Generator(device=dev)
    gen.manual_seed(61)
    pages = L_max // 64
    bt = i32(np.arange(pages, dtype=np.int32)[None, :])
    lens = i32([L_max])
    seq0 = i32([0])

    def fp8_cache(width):
        pool = torch.empty((pages, 64, width), dtype=torch.uint8, device=dev)
        sc = torch.empty((pages, 64, width // 128), dtype=torch.float32, device=dev)
        c = B.LatentCache(pool, bt, lens, sc)
        rows = torch.randn((L_max, width), generator=gen, device=dev).to(bf)
        B.append_latent(c, rows, i32(np.zeros(L_max)), i32(np.arange(L_max)))
        return c

    keys = {l: fp8_cache(d) for l in range(n_layers)}
    lat = [fp8_cache(r) for _ in range(n_groups)]
    q = [torch.randn((1, H, d), generator=gen, device=dev).to(bf) for _ in range(n_layers)]
    W = [(torch.randn((d, r), generator=gen, device=dev) / 16.0).to(bf) for _ in range(n_layers)]
    w = [torch.nn.functional.softplus(torch.randn((1, H), generator=gen, device=dev)) for _ in range(n_layers)]
    new_key = torch.randn((1, d), generator=gen, device=dev).to(bf)
    new_lat = torch.randn((1, r), generator=gen, device=dev).to(bf)
    models = {name: IndexerModel(lm, keys, lat[:len(lm.groups)], q, W, w, k, M, L_max, fp8=True)
              for name, lm in maps.items()}
    torch.cuda.synchronize()

    def run(model, method, Lc, pos):
        model.step(method, seq0, pos, Lc, new_keys={l: new_key for l in range(n_layers)},
                   new_latents={gi: new_lat for gi in range(len(model.lmap.groups))}, new_seq=seq0, new_pos=pos)

    res, res8 = {}, {}
    for Lc in (8192, 32768, 131072):
        pos = i32([Lc - 1])
        ms, ms8 = {}, {}
        for method in ("dsa", "latentindex", "hs", "indexcache"):
            gr = capture(lambda: run(models["G4"], method, Lc, pos))
            ms[method] = time_graph(gr, reps)
            del gr
            if method != "dsa":  # the same work under either map
                gr = capture(lambda: run(models["G8"], method, Lc, pos))
                ms8[method] = time_graph(gr, reps)
                del gr
        res[str(Lc)] = {f"{m}_ms": round(v, 4) for m, v in ms.items()}
        res8[str(Lc)] = {f"{m}_ms": round(v, 4) for m, v in ms8.items()}
        for m in ("latentindex", "hs", "indexcache"):
            res[str(Lc)][f"{m}_speedup_vs_dsa"] = round(ms["dsa"] / ms[m], 3)
            res8[str(Lc)][f"{m}_speedup_vs_dsa"] = round(ms["dsa"] / ms8[m], 3)
    del keys, lat, models
    torch.cuda.empty_cache()
    return {"layer_map": f"{n_layers} layers: layer 0 independent + 15 groups of 4 (FP8 caches; native "
                         f"keys {d} wide, latents {r} wide; H={H}, k={k}, M={M}, batch 1)",
            "per_step": res,
            "layer_map_g8": "layer 0 independent + 7 groups of 8 + 1 group of 4, otherwise the same",
            "per_step_g8": res8,
            "context_from_the_pages": "HS 2.30-2.72x over native DSA decode indexer time across 8K-128K, measured "
                                      "by the pages on 8 GPUs (TP = 8; another machine; context only)"}


def device_facts(dev) -> dict:
    """What the runtime reports about the GPU, and the published peaks every
    fraction in the line is taken against."""
    import torch
    p = torch.cuda.get_device_properties(dev)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "memory_GiB": round(p.total_memory / 2**30, 1), "l2_bytes": getattr(p, "L2_cache_size", None),
            "peaks_used": {"hbm_GBs": HBM_PEAK_GBS, "bf16_dense_TFLOPs": BF16_PEAK_TFLOPS,
                           "fp8_dense_TFLOPs": FP8_PEAK_TFLOPS}}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def source_digest(source: str) -> str:
    """sha256 of a kernel's translation unit as written here: the source file
    and every header it includes with #include "..." from the same folder,
    transitively, taken in name order, each as its name, a NUL byte and its
    bytes.  A counter summary recorded against this digest stays valid only
    while none of those files changes."""
    import hashlib
    import re
    folder = os.path.dirname(source)
    seen, todo = set(), [os.path.basename(source)]
    while todo:
        name = todo.pop()
        if name in seen:
            continue
        seen.add(name)
        with open(os.path.join(folder, name), "rb") as f:
            text = f.read()
        for inc in re.findall(rb'^\s*#\s*include\s+"([^"/]+)"', text, re.M):
            if os.path.exists(os.path.join(folder, inc.decode())):
                todo.append(inc.decode())
    h = hashlib.sha256()
    for name in sorted(seen):
        with open(os.path.join(folder, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(path: str, source: str):
    """HBM bytes per launch of the decode scoring kernel, from a committed
    counter summary, or None when that summary was taken on other kernel
    source (its recorded digest of the kernel's translation unit no longer
    matches) or is absent."""
    try:
        sha = source_digest(source)
        fields = {}
        with open(path) as f:
            for line in f:
                if line.startswith("- ") and ": " in line:
                    key, val = line[2:].split(": ", 1)
                    fields[key.strip()] = val.strip().strip("`")
        if fields.get("source_digest") != sha:
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


class PrefillLayer:
    """Chunked prefill of one layer: 4096 queries at the last positions of a
    `n`-row cache (n = 65536 by default), absorb + score + per-row top-k."""

    def __init__(self, B, synth, dev, bf, i32, tdev, n, fp8=False):
        import numpy as np
        import torch
        self.n, self.Q, self.fp8 = n, 4096, fp8
        p5 = synth.make_prefill("prefill", 5, N=n, Qn=self.Q, r=256, H=64, d=128, G=1, k=2048)
        self.cache = make_cache_from(p5, B, tdev, i32, bf, dev, fp8=fp8)
        self.seq, self.pos = i32(p5.qseq), i32(p5.qpos)
        self.q, self.W, self.w = tdev(p5.q[0], bf), tdev(p5.W[0], bf), torch.from_numpy(p5.w[0]).to(dev)
        if fp8:
            self.qt = B.absorb_query(self.q, self.W, fp8=True)
        else:
            self.qt = torch.empty((p5.Q, p5.H, p5.r), dtype=bf, device=dev)
        self.ws = B.workspace(B.workspace_bytes(B.LI_OP_SCORE_TOPK, p5.Q, n, p5.H, p5.r, p5.k, 0), dev)
        self.out = B.TopK(torch.empty((p5.Q, p5.k), dtype=torch.int32, device=dev),
                          torch.empty(p5.Q, dtype=torch.int32, device=dev))
        self.k = p5.k
        self.pairs = int(np.sum(np.minimum(p5.qpos.astype(np.int64) + 1, n)))
        self.B = B
        self.bias = None  # optional [Q][H] decoder bias

    def layer(self):
        self.B.absorb_query(self.q, self.W, out=self.qt, fp8=self.fp8)
        self.B.score_topk(self.cache, self.seq, self.pos, self.n, self.qt, self.w, self.k, ws=self.ws, out=self.out,
                          bias=self.bias)


def setup_prefill(B, synth, dev, bf, i32, tdev, n, fp8=False):
    return PrefillLayer(B, synth, dev, bf, i32, tdev, n, fp8=fp8)


def make_cache_from(g, B, tdev, i32, bf, dev, fp8=False):
    import numpy as np
    import torch
    if fp8:
        pool = torch.zeros((g.num_pages, 64, g.r), dtype=torch.uint8, device=dev)
        scales = torch.zeros((g.num_pages, 64, g.r // 128), dtype=torch.float32, device=dev)
        c = B.LatentCache(pool, i32(g.block_table), i32(g.lens), scales)
    else:
        pool = torch.zeros((g.num_pages, 64, g.r), dtype=bf, device=dev)
        c = B.LatentCache(pool, i32(g.block_table), i32(g.lens))
    for b in range(g.B):
        n = int(g.lens[b])
        B.append_latent(c, tdev(g.latent[b], bf), i32(np.full(n, b)), i32(np.arange(n)))
    return c


if __name__ == "__main__":
    sys.exit(main())

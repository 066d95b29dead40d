// The tail of the decode scoring kernels (gfx950): the staged scores leave
// in one pass per workgroup, which also counts their first radix digit, and
// optionally the filter pass of the top-k selection runs right there, on
// the scores the workgroup still holds in LDS.
//
// LatentIndex (paperlayer.ai summary of arXiv:2610.04635), §3.1/§4.1 and
// §C.4: each layer keeps its own top-k rows of the valid prefix (the HS
// anchor its top-M and, nested in them, its top-k).  The selection is a
// radix select on order-preserving keys; its first pass finds the digit on
// which the k-th largest key lies (from the query's first-digit histogram)
// and splits the rows into those above it (selected) and those on it (tied,
// resolved later by the remaining digits).
#pragma once

#include "li_device.hpp"
#include "li_internal.hpp"
#include "li_radix.hpp"

namespace li {
namespace {

// LDS scratch of the fused filter pass, carved from the chunk ring (which
// the stream no longer uses by then).
struct FilterLds {
    uint32_t wtot[4];
    int res[4];
    int cnt[4];
    int base[4];
    int err;
};



// Loads and adds at agent scope: performed where every XCD sees them (not in
// this XCD's L2), so workgroups on different XCDs exchange counts without a
// cache writeback or invalidate.
__device__ __forceinline__ int load_agent(int32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int add_agent(int32_t *p, int v)
{
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The per-call counters of query q's entry in the workspace's zeroed region
// (rows above and on the threshold digits, rows sorted), zeroed by the
// scoring kernel's first workgroup before it counts its own rows: no
// workgroup uses them before the query's histogram is complete, which needs
// that workgroup's rows, so the zeroes land first.  Thread 0 of workgroup 0.
__device__ __forceinline__ void zero_filter_counters(int32_t *hq)
{
    const int slots[5] = {kSlotUpO, kSlotTieO, kSlotUpI, kSlotTieI, kSlotDone};
#pragma unroll
    for (int i = 0; i < 5; ++i) __hip_atomic_store(hq + slots[i], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Rows per thread per round of the tail's passes over the staged scores
// (2048 of a workgroup's rows): a round's LDS reads go out together, which
// matters here, where each SIMD runs one wave.
constexpr int kTailU = 8;

// Scores of rows c0 + u * 256 + tid (u < kTailU) of the workgroup's rows
// (reads past the last row repeat it; live[u] says which rows are real).
__device__ __forceinline__ void tail_round(const lds_f32 *s_out, int c0, int rows, float (&p)[kTailU],
                                           bool (&live)[kTailU])
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < kTailU; ++u) {
        const int j = c0 + u * 256 + tid;
        live[u] = j < rows;
        p[u] = s_out[min(j, rows - 1)];
    }
}

// The filter pass over this workgroup's rows row0 .. row0 + rows - 1 of
// query q (n rows in all, rows >= 1), their scores in s_out; the
// workgroup's digit counts and its row count are already being added into
// the query's histogram hq and its row total (all 256 threads).
__device__ __forceinline__ void filter_pass(const ScoreArgs &a, int q, int64_t row0, int rows, int n,
                                            const lds_f32 *s_out, uint32_t *s_hist, int32_t *hq, FilterLds *fl)
{
    const int tid = threadIdx.x, lane = tid & 63;
    const FilterArgs &f = a.flt;
    const int K = min(n, f.k);
    const int Ki = f.k_inner > 0 ? min(n, f.k_inner) : 0;
    const uint32_t rem[2] = {(uint32_t)K, (uint32_t)(Ki > 0 ? Ki : K)};
    if (tid < 4) fl->cnt[tid] = 0;
    // The workgroup whose row count completes the query's row total (its
    // add returns n - rows) finds the threshold digits for all of them:
    // every other workgroup has issued its histogram adds by then, and a
    // histogram whose bins sum to n holds every add (no bin reads more than
    // its final count), so a sum short of n is read again.  It publishes the
    // digits in one 64-bit word (with a flag and the row count n), which the
    // other workgroups poll.  Only agent-scope loads, adds and stores are used:
    // no cache writeback or invalidate.  The launcher fuses the pass only
    // when the whole grid fits the GPU at once, so the wait normally ends
    // within microseconds; it is bounded (f.wait_ticks of the 100 MHz
    // constant clock) because other work can hold CUs meanwhile (another
    // stream's kernels, another fused launch waiting the same way).  A
    // workgroup whose wait runs out leaves its rows unsorted (they are then
    // missing from the query's count of sorted rows), and the final kernel
    // selects that query again from its scores alone.
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    auto expired = [&] { return __builtin_amdgcn_s_memrealtime() - t0 >= f.wait_ticks; };
    uint64_t *res_word = (uint64_t *)(hq + kSlotResult);
    if (tid == 0) fl->err = add_agent(hq + kSlotTotal, rows) + rows == n ? 2 : 0; // 2: this workgroup is last
    __syncthreads();
    if (fl->err == 2) {
        for (;;) {
            constexpr int PB = kHistBins / 256;
            uint32_t hv[PB];
#pragma unroll
            for (int e = 0; e < PB; ++e) hv[e] = (uint32_t)load_agent(hq + e * 256 + tid);
#pragma unroll
            for (int e = 0; e < PB; ++e) s_hist[e * 256 + tid] = hv[e];
            __syncthreads();
            find_bins<256, kHistBins, 2>(s_hist, rem, *fl);
            const uint32_t total = fl->wtot[0] + fl->wtot[1] + fl->wtot[2] + fl->wtot[3];
            if (total == (uint32_t)n) break;
            __syncthreads(); // every thread has read this round's results
            if (tid == 0) fl->err = expired() ? 1 : 2;
            __syncthreads();
            if (fl->err == 1) break;
        }
        if (tid == 0) {
            if (fl->err != 1) {
                // for the final kernel, then for the other workgroups
                hq[kSlotBins] = (int32_t)(((uint32_t)fl->res[0] & 0xFFFFu) | ((uint32_t)fl->res[2] << 16));
                hq[kSlotAboveO] = fl->res[1];
                hq[kSlotAboveI] = fl->res[3];
                const uint64_t w = (1ull << 63) | ((uint64_t)(uint32_t)n << 26) |
                                   (uint64_t)(uint32_t)(fl->res[0] + 1) | ((uint64_t)(uint32_t)(fl->res[2] + 1) << 13);
                __hip_atomic_store(res_word, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                fl->err = 0;
            }
        }
    } else if (tid == 0) {
        uint64_t w = 0;
        int err = 0;
        // the word is this call's once its flag is set and it names this
        // query's row count (a workspace that was not zeroed may hold any bits)
        const uint64_t want = (1ull << 63) | ((uint64_t)(uint32_t)n << 26);
        while (((w = __hip_atomic_load(res_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) & ~0x3FFFFFFull) !=
               want) {
            __builtin_amdgcn_s_sleep(2);
            if (expired()) {
                err = 1;
                break;
            }
        }
        fl->err = err;
        fl->res[0] = (int)(w & 0x1FFFu) - 1;
        fl->res[2] = (int)((w >> 13) & 0x1FFFu) - 1;
    }
    __syncthreads();
    if (fl->err) return;
    const int bin = fl->res[0];
    const int bin_i = Ki > 0 ? fl->res[2] : -1;
    if (bin < 0 || (Ki > 0 && bin_i < 0)) return; // inconsistent counts
    const bool inner = Ki > 0;
    const bool sep = inner && bin_i != bin; // inner ties need a list of their own
    // a row's runs: above the outer digit (0) or on it (1), above the inner
    // digit (2) or on it when that differs from the outer one (3); dg = -1
    // for reads past the last row, which lie in no run
    auto runs = [&](int dg, bool (&in)[4]) {
        in[0] = dg > bin;
        in[1] = dg == bin;
        in[2] = inner && dg > bin_i;
        in[3] = sep && dg == bin_i;
    };
    const int lo = inner ? min(bin, bin_i) : bin; // rows below this digit lie in no run
    // Pass 1: each wave counts its rows in every run (ballots), takes its
    // offsets in the workgroup's runs with one LDS add per run, and the
    // workgroup's totals go to the query's run counters in one global add
    // each, whose results (the workgroup's bases) are waited for only after
    // pass 2 has ranked the first round's rows.
    uint32_t wcnt[4] = {0u, 0u, 0u, 0u};
    for (int c0 = 0; c0 < rows; c0 += 256 * kTailU) {
        float p[kTailU];
        bool live[kTailU];
        tail_round(s_out, c0, rows, p, live);
#pragma unroll
        for (int u = 0; u < kTailU; ++u) {
            const int dg = live[u] ? (int)(score_key(p[u]) >> kDigit0Shift) : -1;
            if (__ballot(dg >= lo) == 0) continue; // the usual round: no row of the wave in a run
            bool in[4];
            runs(dg, in);
#pragma unroll
            for (int r = 0; r < 4; ++r) wcnt[r] += (uint32_t)__popcll(__ballot(in[r]));
        }
    }
    uint32_t woff[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        int v = 0;
        if (lane == 0 && wcnt[r]) v = atomicAdd(&fl->cnt[r], (int)wcnt[r]);
        woff[r] = (uint32_t)__builtin_amdgcn_readfirstlane(v);
    }
    __syncthreads(); // the workgroup's run totals are complete
    int gbase = 0;
    if (tid < 4) {
        const int slot = tid == 0 ? kSlotUpO : tid == 1 ? kSlotTieO : tid == 2 ? kSlotUpI : kSlotTieI;
        const int v = fl->cnt[tid];
        if (v) gbase = add_agent(hq + slot, v);
    }
    // Pass 2: every row of a run gets its slot (the wave's offset, the rows
    // of earlier rounds, then lane order) and is stored there: out / outi
    // hold row ids, cand / cand2 (key, row id) pairs; slots past a list's
    // end are dropped but still counted.
    int32_t *out = f.idx + (int64_t)q * f.k;
    int32_t *outi = inner ? f.idx_inner + (int64_t)q * f.k_inner : nullptr;
    uint2 *cand = f.cand + (int64_t)q * f.cap;
    uint2 *cand2 = f.cand2 + (int64_t)q * f.cap;
    const uint64_t below = lanes_below();
    for (int c0 = 0; c0 < rows; c0 += 256 * kTailU) {
        float p[kTailU];
        bool live[kTailU];
        tail_round(s_out, c0, rows, p, live);
        int slot[kTailU][2]; // the row's slot in its outer run (0 or 1) and in its inner run (2 or 3)
        int dgs[kTailU];
#pragma unroll
        for (int u = 0; u < kTailU; ++u) {
            const int dg = live[u] ? (int)(score_key(p[u]) >> kDigit0Shift) : -1;
            dgs[u] = dg;
            slot[u][0] = slot[u][1] = 0;
            if (__ballot(dg >= lo) == 0) continue;
            bool in[4];
            runs(dg, in);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint64_t m = __ballot(in[r]);
                if (in[r]) slot[u][r >> 1] = (int)(woff[r] + (uint32_t)__popcll(m & below));
                woff[r] += (uint32_t)__popcll(m);
            }
        }
        if (c0 == 0) {
            if (tid < 4) fl->base[tid] = gbase;
            __syncthreads(); // the workgroup's bases
        }
        const int b0 = fl->base[0], b1 = fl->base[1], b2 = fl->base[2], b3 = fl->base[3];
#pragma unroll
        for (int u = 0; u < kTailU; ++u) {
            const int dg = dgs[u];
            if (dg < lo) continue;
            const int32_t i = (int32_t)(row0 + c0 + u * 256 + tid);
            if (dg > bin) {
                const int s = b0 + slot[u][0];
                if (s < f.k) out[s] = i;
            } else if (dg == bin) {
                const int s = b1 + slot[u][0];
                if (s < f.cap) cand[s] = make_uint2(score_key(p[u]), (uint32_t)i);
            }
            if (inner) {
                if (dg > bin_i) {
                    const int s = b2 + slot[u][1];
                    if (s < f.k_inner) outi[s] = i;
                } else if (sep && dg == bin_i) {
                    const int s = b3 + slot[u][1];
                    if (s < f.cap) cand2[s] = make_uint2(score_key(p[u]), (uint32_t)i);
                }
            }
        }
    }
    if (tid == 0) add_agent(hq + kSlotDone, rows); // this workgroup's rows are sorted
}

// After the stream, with every row's score staged in s_out (workgroup-local
// row j is row row0 + j of query q, j < rows): the scores leave in one
// coalesced pass; with a histogram, their first radix digits are counted in
// LDS and merged into the query's histogram (non-empty bins only), and with
// the fused filter pass the scores leave after it (nothing in this launch
// reads them).  A workgroup past the query's last row (rows <= 0) has
// nothing to count or sort and takes no part in the filter pass, whose row
// total is then the sum of the others' rows, n.  All 256 threads.
__device__ __forceinline__ void score_tail(const ScoreArgs &a, int q, int64_t row0, int rows, int n,
                                           const lds_f32 *s_out, uint32_t *s_hist, FilterLds *fl)
{
    if (rows <= 0) return;
    const int tid = threadIdx.x;
    float *out = a.out + (int64_t)q * a.out_ld + row0;
    auto store_scores = [&] {
        for (int c0 = 0; c0 < rows; c0 += 256 * kTailU) {
            float p[kTailU];
            bool live[kTailU];
            tail_round(s_out, c0, rows, p, live);
#pragma unroll
            for (int u = 0; u < kTailU; ++u)
                if (live[u]) out[c0 + u * 256 + tid] = p[u];
        }
    };
    if (!a.hist) {
        store_scores();
        return;
    }
    int32_t *hq = a.hist + (int64_t)q * kHistStride;
    const bool fused = a.flt.on;
    for (int c0 = 0; c0 < rows; c0 += 256 * kTailU) {
        float p[kTailU];
        bool live[kTailU];
        tail_round(s_out, c0, rows, p, live);
#pragma unroll
        for (int u = 0; u < kTailU; ++u) {
            if (!live[u]) continue;
            if (!fused) out[c0 + u * 256 + tid] = p[u];
            atomicAdd(&s_hist[score_key(p[u]) >> kDigit0Shift], 1u);
        }
    }
    __syncthreads();
    hist_flush(s_hist, hq, 256, tid);
    if (!fused) return;
    __syncthreads(); // every thread has issued its adds (and read s_hist, which the filter pass reuses)
    filter_pass(a, q, row0, rows, n, s_out, s_hist, hq, fl);
    store_scores();
}

} // namespace
} // namespace li

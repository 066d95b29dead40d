// Host-side launchers shared between the translation units of liblatentindex.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "li_common.hpp"

namespace li {

constexpr int kHistBins = 4096;   // first radix digit: key bits [31:20]
constexpr int kHistStride = kHistBins + 16; // per query: histogram, then the slots below
constexpr int kSelThreads = 1024; // threads of the per-query selection workgroup

// Per-query slots after the histogram.
enum {
    kSlotUpO = kHistBins + 0,  // rows emitted above the outer threshold digit (filter counter)
    kSlotTieO = kHistBins + 1, // rows on the outer threshold digit (filter counter)
    kSlotN = kHistBins + 2,    // the query's row count, recorded by the scoring kernel
    kSlotUpI = kHistBins + 3,  // same two counters for the nested (inner) selection
    kSlotTieI = kHistBins + 4,
    kSlotBins = kHistBins + 5,   // threshold digits found by the filter: outer | inner << 16 (-1: none)
    kSlotAboveO = kHistBins + 6, // rows in digits above the outer threshold digit
    kSlotAboveI = kHistBins + 7, // the same for the inner one
    kSlotTotal = kHistBins + 8,  // rows counted into the histogram so far (fused filter pass)
    kSlotDone = kHistBins + 9,   // rows the filter pass has sorted (short of n: the final kernel redoes the query)
    kSlotResult = kHistBins + 10, // 64-bit (slots 10, 11): threshold digits published by the fused filter pass
};

// The long-row selection's filter path (at most kSyncQueries queries) keeps
// each query's histogram and counters in a region at the start of the
// workspace, which is zero between calls: the final kernel clears what a
// call added to it (the histogram, the row total, the published digits), and
// the scoring kernel's first workgroup zeroes the per-call counters before
// any workgroup can use them, so no kernel has to clear the histogram before
// scoring.
constexpr int kSyncQueries = 64;
constexpr size_t kSyncBytes = ((size_t)kSyncQueries * kHistStride * 4 + 255) & ~(size_t)255;

// The filter pass of a long-row selection, run inside the decode scoring
// kernel (on: the launcher guarantees that every workgroup of the grid is
// resident at once).  Once every workgroup of a query has added its scores'
// first digits to the histogram, each one finds the threshold digits from it
// and emits, from the scores it holds in LDS, its rows above them to idx /
// idx_inner and its rows on them to the tie lists cand / cand2 (the
// selection's workspace), as the separate filter kernel would.
struct FilterArgs {
    bool on;
    bool filter_path; // the selection takes the filter path: the histogram is the
                      // query's entry in the workspace's zeroed region, and the
                      // scoring kernel's first workgroup zeroes the per-call counters
    int32_t k;
    int32_t k_inner; // 0: no nested selection
    int32_t *idx;    // [Q][k]
    int32_t *idx_inner;
    uint2 *cand; // [Q][cap]
    uint2 *cand2;
    int64_t cap;
    uint32_t wait_ticks; // bound on the wait for the query's histogram (100 MHz clock ticks)
};

// Geometry of a paged pool, for bounding device-resident indices.
struct PoolGeom {
    int32_t batch;
    int32_t max_pages;
    int32_t num_pages;
    // Physical row of position p of sequence s, or -1 when s, p or the page
    // they map to lies outside the cache.
    __device__ __forceinline__ int64_t slot(const int32_t *bt, int s, int p) const
    {
        if (s < 0 || s >= batch || p < 0 || (int64_t)p >= (int64_t)max_pages * 64) return -1;
        const int page = bt[(int64_t)s * max_pages + (p >> 6)];
        if (page < 0 || page >= num_pages) return -1;
        return (int64_t)page * 64 + (p & 63);
    }
};

// Rows to score for one call.
//   contiguous mode (cand == nullptr): query i scores its causal prefix
//     rows 0..n_i-1, n_i = min(qpos[i] + 1, seq_lens[qseq[i]]);
//   gather mode: query i scores rows cand[i*cand_ld + j], j < min(cand_count[i], cand_ld).
// out[i*out_ld + j] receives the score of the j-th row of query i.
struct ScoreArgs {
    const void *pool;
    const int32_t *bt;
    int32_t max_pages;
    int32_t num_pages; // pages in the pool (page ids read ahead of the row count are clamped to it)
    int32_t batch;     // sequences in the block table
    const int32_t *seq_lens;
    const int32_t *qseq;
    const int32_t *qpos;
    const int32_t *cand;
    const int32_t *cand_count;
    int64_t cand_ld;
    const void *qt;
    const float *w;
    const float *bias; // optional [Q][H]: absorbed decoder bias, added before the ReLU
    int32_t H;
    int32_t Q;
    float *out;
    int64_t out_ld;
    int64_t max_rows; // bound on every query's row count (rows past it are not scored)
    int32_t *hist;    // optional [Q][kHistStride]: first-digit counts of the keys written
                      // (accumulated) and the query's row count in slot kSlotN
    bool stream_nt;   // latent rows are read with the non-temporal policy (not kept in the caches)
    FilterArgs flt;   // optional fused filter pass (contiguous decode with a histogram only)
};

// Scoring.  `max_rows` bounds every query's row count (grid sizing).
// filtered (optional): set to whether the launch ran the fused filter pass
// that a.flt asked for (the selection then skips its own filter kernel).
hipError_t launch_score(const ScoreArgs &a, int r, bool bf16, bool many_queries_per_seq,
                        int64_t max_rows, hipStream_t s, bool *filtered = nullptr);

// Compute units of the current device (0 if unknown), and whether a decode
// scoring grid of wgs_per_query x Q workgroups is resident all at once.
int device_cu_count();
bool fused_filter_fits(int64_t wgs_per_query, int64_t Q);

// out[q][j] = S[q][cand[q][j]] for j < min(cand_count[q], M) (candidates
// clamped into [0, ld)); entries past the count are left untouched.
hipError_t launch_gather_scores(const float *S, int64_t ld, const int32_t *cand, const int32_t *cand_count, int64_t M,
                                float *out, int32_t Q, hipStream_t s);

// Absorption qt = q W (see li_absorb_query).
hipError_t launch_absorb(const void *q, const void *W, void *qt, int64_t QH, int d, int r, bool bf16,
                         hipStream_t s);

// Segmented FP8: query buffer layout, append (rotate + quantize), absorption
// into FP8, and FP8 scoring (the prefill kernel when many queries share a
// sequence and no histogram is asked for; the decode kernel otherwise).
int64_t fp8_query_scale_offset(int64_t Q, int64_t H, int64_t r);
// Rotary layout of a latent row (see li_rope): F frequencies, S sources, and
// the phase step theta_f of each frequency (computed on the host in fp64).
constexpr int kMaxRopeFreqs = 64;
struct RopeArgs {
    int32_t F; // 0: no rotary part
    int32_t S;
    double theta[kMaxRopeFreqs];
};

hipError_t launch_append_fp8(void *pool, float *scales, const int32_t *bt, const PoolGeom &geo, int r, const void *rows,
                             const int32_t *seq, const int32_t *pos, int T, const RopeArgs &rope, hipStream_t s);
hipError_t launch_absorb_fp8(const void *q, const void *W, void *qt, int64_t QH, int d, int r, hipStream_t s);
hipError_t launch_score_fp8(const ScoreArgs &a, const float *pool_scales, int64_t qscale_off, int r,
                            bool many_queries_per_seq, int64_t max_rows, hipStream_t s, bool *filtered = nullptr);

// Append rows into the paged pool.
hipError_t launch_append(void *pool, const int32_t *bt, const PoolGeom &geo, int r, int esize, const void *rows,
                         const int32_t *seq, const int32_t *pos, int T, hipStream_t s);

// RoPE-compatible structured decoder: rotated append (bf16 / fp32 pools),
// lowering of the decoder to a dense W, and the absorbed bias.
hipError_t launch_append_rope(void *pool, const int32_t *bt, const PoolGeom &geo, int r, int esize, const void *rows,
                              const int32_t *seq, const int32_t *pos, int T, const RopeArgs &rope, hipStream_t s);
hipError_t launch_rope_decoder(const void *D, const void *Wn, int F, int S, int d_nope, int r_nope, void *W, int esize,
                               hipStream_t s);
hipError_t launch_query_bias(const void *q, const float *beta, int64_t QH, int d, int d_rope, float *bias, bool bf16,
                             hipStream_t s);

// ---------------------------------------------------------------------------
// Top-k selection over per-query virtual rows of scores.
// ---------------------------------------------------------------------------
struct SelWorkspace {
    int32_t *hist; // [Q][kHistStride]: first-digit counts, then the slots above
    uint2 *cand;   // [Q][cap] (key, index) of rows tied on the threshold digit
    uint2 *cand2;  // [Q][cap] the same for the nested selection's threshold digit
    int64_t cap;
};

// How the per-query element count is found:
//   kSrcCausal: n = min(qpos+1, seq_lens[qseq])
//   kSrcCount : n = min(cnt[q], cnt_cap)
enum { kSrcCausal = 0, kSrcCount = 1 };

struct SelCall {
    SelRow row;
    int src_mode;
    const int32_t *qseq, *qpos, *seq_lens;  // kSrcCausal
    int32_t batch;                           // sequences (qseq entries are clamped below it)
    const int32_t *cnt;                      // kSrcCount
    int32_t cnt_cap;
    int32_t Q;
    int32_t k;
    int64_t max_n;   // host bound on every n
    int32_t *idx;    // [Q][k]
    int32_t *count;  // [Q]
    // Optional nested selection (k_inner > 0): the top-k_inner rows, always a
    // subset of the top-k ones.
    int32_t k_inner;
    int32_t *idx_inner;   // [Q][k_inner]
    int32_t *count_inner; // [Q]
};

size_t sel_workspace_bytes(int64_t Q, int64_t max_n);
// base: the workspace past its zeroed region sync (the filter path's
// histograms, when the selection takes that path).
SelWorkspace sel_workspace_carve(void *base, int64_t Q, int64_t max_n, int32_t *sync);

// Zero the histograms (before a scoring kernel accumulates into them).
hipError_t launch_hist_clear(const SelWorkspace &ws, int64_t Q, hipStream_t s);
// The selection proper (after scores exist).  have_hist: a scoring kernel
// filled ws.hist (histogram and row counts) for these very scores; filtered:
// it also ran the filter pass (ScoreArgs::flt), so only the tie resolution
// is left.
hipError_t launch_select(const SelCall &c, const SelWorkspace &ws, bool have_hist, hipStream_t s,
                         bool filtered = false);

// Whether the selection of Q queries over rows of up to max_n scores takes
// the filter path (many workgroups per query, then the tie resolution),
// whose filter pass a decode scoring kernel can run (ScoreArgs::flt).
bool selection_filters(int64_t Q, int64_t max_n);

// Whether a selection of Q queries over rows of up to max_n scores wants the
// scoring kernel to count the first radix digit: rows of up to 8192 scores,
// and those of up to 16384 for at most 64 queries, are counted by the
// one-workgroup selection from the keys it holds anyway, which costs less
// than clearing the histogram in a kernel of its own; longer rows are
// counted by the scoring kernel.
bool selection_wants_counts(int64_t Q, int64_t max_n);

} // namespace li

// Per-query top-k selection (gfx950).
//
// LatentIndex (paperlayer.ai summary of arXiv:2610.04635), §3.1/§4.1: every
// layer picks its own top-k rows (k = 2048), capped by the valid prefix
// (§C.4); the HS anchor picks its top-M candidates and its own top-k inside
// them (§3.2, §C.4).
//
// Scores become order-preserving uint32 keys, selected by radix digits of
// 12, 11 and 9 bits (most significant first).  For rows longer than 8192
// the decode scoring kernels already count the first digit (key >> 20)
// into a per-query 4096-bin histogram as they write the scores, and record
// the row count beside it, so the threshold bin is known before the rows
// are read again; otherwise the selection counts it itself.  One pass over each row then emits the
// rows above the threshold digit and compacts the rows on it; the last two
// digits are resolved among those few in LDS.
//   * Few queries with long rows (decode at 8K-128K): the pass is spread
//     over many workgroups per query (k_filter), and one workgroup per
//     query finishes (k_final).  A nested selection (the HS anchor's top-k
//     inside its top-M) rides along in the same two kernels.
//   * Many queries or short rows (prefill, HS followers, the anchor's nested
//     selection elsewhere): one 1024-thread workgroup per query does it all
//     (k_select); rows of at most 8192 elements are loaded once, up front.
// Every kernel issues all of its input loads before its first wait (rows
// are read 16 bytes per lane; the scores were written by other XCDs, so
// each load misses the local L2).  The kernels are chains of short
// dependent steps, so the steps are few: threshold searches scan with DPP
// (no LDS permutes), and emission ranks lanes with ballots and popcounts
// under one LDS atomic per wave for all of a thread's elements.  Rows whose
// key equals the final threshold key are taken in element order, as many as
// the budget needs: equal scores are interchangeable, and the fixed order
// keeps nested selections nested.
#include "li_internal.hpp"
#include "li_radix.hpp"

#include <algorithm>

namespace li {
namespace {

constexpr int NT = kSelThreads;
constexpr int kB = 4;              // 16-byte loads in flight per thread per round
constexpr int kCandCap = 8192;     // tied rows kept in LDS
constexpr int kKeyCache = 16384;   // rows cached in LDS when the histogram is built here
constexpr int kFilterThreads = 256;
constexpr int kFilterChunk = kFilterThreads * kB * 4; // rows per filter workgroup (4096)

__device__ __forceinline__ uint32_t key_at(const SelRow &r, int q, int64_t i)
{
    int64_t j = i;
    if (r.gmap) { // a mapped index stays inside the row
        j = r.gmap[(int64_t)q * r.gld + i];
        j = j < 0 ? 0 : (j < r.ld ? j : r.ld - 1);
    }
    return score_key(r.S[(int64_t)q * r.ld + j]);
}

// Keys of rows i..i+3 (zero past n).
__device__ __forceinline__ void keys4(const SelRow &r, int q, int64_t i, int64_t n, uint32_t (&k)[4])
{
    if (!r.gmap && (r.ld & 3) == 0 && i + 3 < n) {
        const float4 v = *(const float4 *)(r.S + (int64_t)q * r.ld + i);
        k[0] = score_key(v.x);
        k[1] = score_key(v.y);
        k[2] = score_key(v.z);
        k[3] = score_key(v.w);
    } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) k[t] = i + t < n ? key_at(r, q, i + t) : 0u;
    }
}

__device__ __forceinline__ int32_t out_id(const SelRow &r, int q, int64_t i)
{
    return r.omap ? r.omap[(int64_t)q * r.old + i] : (int32_t)i;
}

__device__ __forceinline__ int clamp_n(int n, int64_t max_n)
{
    n = n > 0 ? n : 0;
    return n < max_n ? n : (int)max_n; // the caller's bound sizes every buffer
}

// Row count of query q computed from the call's own inputs (used when no
// scoring kernel recorded it).
__device__ __forceinline__ int query_n(const SelCall &c, int q)
{
    int n;
    if (c.src_mode == kSrcCausal) {
        n = valid_rows(c.qpos[q], c.seq_lens[clamp_index(c.qseq[q], c.batch)]);
    } else {
        n = c.cnt[q] < c.cnt_cap ? c.cnt[q] : c.cnt_cap;
    }
    return clamp_n(n, c.max_n);
}

// Smallest and largest of x over the wave (unsigned), in every lane: DPP
// row shifts leave each row's extreme in its last lane (a lane without a
// source keeps its own value), and the four rows are combined by readlane.
__device__ __forceinline__ void wave_min_max(uint32_t &lo, uint32_t &hi)
{
#define LI_MINMAX_STEP(ctrl)                                                                     \
    lo = min(lo, (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, ctrl, 0xf, 0xf, false)); \
    hi = max(hi, (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, ctrl, 0xf, 0xf, false));
    LI_MINMAX_STEP(0x111) // row_shr:1
    LI_MINMAX_STEP(0x112) // row_shr:2
    LI_MINMAX_STEP(0x114) // row_shr:4
    LI_MINMAX_STEP(0x118) // row_shr:8
#undef LI_MINMAX_STEP
    uint32_t l = (uint32_t)__builtin_amdgcn_readlane((int)lo, 15);
    uint32_t h = (uint32_t)__builtin_amdgcn_readlane((int)hi, 15);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
        l = min(l, (uint32_t)__builtin_amdgcn_readlane((int)lo, 16 * r + 15));
        h = max(h, (uint32_t)__builtin_amdgcn_readlane((int)hi, 16 * r + 15));
    }
    lo = l;
    hi = h;
}

template <int T>
struct Scratch {
    uint32_t hist[2048]; // second digit, bits [19:9]
    uint32_t hist2[512]; // third digit, bits [8:0]
    uint32_t wtot[T / 64];
    uint32_t wlo[T / 64]; // per-wave key range (short-row selection)
    uint32_t whi[T / 64];
    int few[64]; // element indices of a threshold digit holding at most 64 elements
    int res[4];
    int cnt[4];
    // Both level histograms start at zero; visible after the caller's next barrier.
    __device__ __forceinline__ void clear_levels()
    {
        for (int j = threadIdx.x; j < 2048 + 512; j += T) (j < 2048 ? hist[j] : hist2[j - 2048]) = 0;
    }
};

// The first-digit histogram of one query, held in registers between its
// (early) load and its store into LDS.
template <int T>
struct HistRegs {
    uint32_t v[kHistBins / T];
    __device__ __forceinline__ void load(const int32_t *g)
    {
#pragma unroll
        for (int e = 0; e < kHistBins / T; ++e) v[e] = (uint32_t)g[e * T + threadIdx.x];
    }
    __device__ __forceinline__ void store(uint32_t *h) const
    {
#pragma unroll
        for (int e = 0; e < kHistBins / T; ++e) h[e * T + threadIdx.x] = v[e];
    }
};

// Compacting append for U rounds at once: lanes with e[u] set get slots
// base + (rank in round order, then lane order) from one LDS atomic per
// wave on *cnt, and store(u, slot) is called for slots below cap (the count
// still grows past cap, so overflow stays visible).  Whole waves must reach it.
template <int U, class Store>
__device__ __forceinline__ void wave_append(const bool (&e)[U], int *cnt, int cap, Store store)
{
    uint64_t m[U];
    int tot = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        m[u] = __ballot(e[u]);
        tot += __popcll(m[u]);
    }
    if (tot == 0) return;
    int base = 0;
    if ((threadIdx.x & 63) == 0) base = atomicAdd(cnt, tot);
    base = __builtin_amdgcn_readfirstlane(base);
    const uint64_t below = lanes_below();
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int slot = base + __popcll(m[u] & below);
        if (e[u] && slot < cap) store(u, slot);
        base += __popcll(m[u]);
    }
}

// Element sources for the in-block levels: key(i) and the id to output.
struct CandLds {
    const uint32_t *k;
    const int32_t *d;
    __device__ uint32_t key(int i) const { return k[i]; }
    __device__ int32_t out(int i) const { return d[i]; }
};
struct CacheLds {
    const uint32_t *k;
    SelRow r;
    int q;
    __device__ uint32_t key(int i) const { return k[i]; }
    __device__ int32_t out(int i) const { return out_id(r, q, i); }
};
struct RowGlobal {
    SelRow r;
    int q;
    __device__ uint32_t key(int i) const { return key_at(r, q, i); }
    __device__ int32_t out(int i) const { return out_id(r, q, i); }
};
// The global tie list a filter pass wrote: (key, row index) pairs.
struct CandGlobal {
    const uint2 *c;
    SelRow r;
    int q;
    __device__ uint32_t key(int i) const { return c[i].x; }
    __device__ int32_t out(int i) const { return out_id(r, q, (int64_t)c[i].y); }
};

// The last step when at most 64 elements are left to choose from: wave 0
// holds one per lane (element list[l], or element l without a list) and
// ranks it by a pass over the other lanes' keys (larger key first, then
// lower element index), so element x is taken iff fewer than `need` live
// elements precede it; its slot is base + rank.  This is the order the
// digit passes give (ties in element order) without their barriers.  Live:
// (key & pmask) == prefix.  Wave 0 only.
template <class Src>
__device__ __forceinline__ void rank_take(const Src &src, int cnt, const int *list, uint32_t prefix, uint32_t pmask,
                                          uint32_t need, int32_t *out, int cap, int base)
{
    const int lane = threadIdx.x & 63;
    const int x = lane < cnt ? (list ? list[lane] : lane) : 0;
    const uint32_t k = lane < cnt ? src.key(x) : 0u;
    const bool live = lane < cnt && (k & pmask) == prefix;
    const uint64_t lm = __ballot(live);
    uint32_t rank = 0;
    for (int j = 0; j < cnt; ++j) {
        const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)k, j);
        const int xj = __builtin_amdgcn_readlane(x, j);
        rank += ((lm >> j) & 1ull) && (kj > k || (kj == k && xj < x)) ? 1u : 0u;
    }
    if (live && rank < need) {
        const int slot = base + (int)rank;
        if (slot < cap) out[slot] = src.out(x);
    }
}

// One digit level over m elements restricted to (key & pmask) == prefix,
// the level's histogram pre-cleared: count, find the threshold digit, emit
// the elements above it at out[sh.cnt[0] ...], then narrow prefix/pmask and
// the budget.  False if the counts are inconsistent.
template <int T, class Src, int U, int SHIFT, int NB>
__device__ __forceinline__ bool digit_level(const Src &src, int m, uint32_t &prefix, uint32_t &pmask,
                                            uint32_t &remaining, int32_t *out, int cap, uint32_t *hist,
                                            Scratch<T> &sh)
{
    const int tid = threadIdx.x, lane = tid & 63;
    const int wbase = tid - lane;
    constexpr uint32_t dmask = (uint32_t)NB - 1u;
    if (tid == 0) sh.cnt[2] = 0; // the short list below; find_bins' barriers publish it
    // U elements per thread per round: their (possibly global) loads go
    // out together before the LDS updates that use them
    for (int i0 = tid; i0 < m; i0 += T * U) {
        uint32_t kk[U];
#pragma unroll
        for (int u = 0; u < U; ++u) kk[u] = i0 + u * T < m ? src.key(i0 + u * T) : 0u;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (i0 + u * T < m && (kk[u] & pmask) == prefix) atomicAdd(&hist[(kk[u] >> SHIFT) & dmask], 1u);
    }
    __syncthreads();
    const uint32_t rem[1] = {remaining};
    find_bins<T, NB, 1>(hist, rem, sh);
    const int bin = sh.res[0];
    const uint32_t above = (uint32_t)sh.res[1];
    if (bin < 0) return false;
    // when the threshold digit holds exactly the elements still needed (the
    // usual case once the list is down to a few hundred), they are all taken
    // here and the next level is skipped
    const bool all = above + hist[bin] == remaining;
    // a threshold digit of at most 64 elements is listed in this pass and
    // ranked in one wave after it, which ends the selection here
    const bool listed = !all && hist[bin] <= 64u;
    for (int i0 = wbase; i0 < m; i0 += T * U) {
        bool e[U], f[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * T + lane;
            const uint32_t k = i < m ? src.key(i) : 0u;
            const uint32_t dg = (k >> SHIFT) & dmask;
            const bool in = i < m && (k & pmask) == prefix;
            e[u] = in && (dg > (uint32_t)bin || (all && dg == (uint32_t)bin));
            f[u] = listed && in && dg == (uint32_t)bin;
        }
        wave_append<U>(e, &sh.cnt[0], cap, [&](int u, int slot) { out[slot] = src.out(i0 + u * T + lane); });
        if (listed) wave_append<U>(f, &sh.cnt[2], 64, [&](int u, int slot) { sh.few[slot] = i0 + u * T + lane; });
    }
    if (all) {
        remaining = 0;
        return true;
    }
    if (listed) {
        __syncthreads(); // the list and the output count are complete
        if (tid < 64)
            rank_take(src, min(sh.cnt[2], 64), sh.few, prefix | ((uint32_t)bin << SHIFT), pmask | (dmask << SHIFT),
                      remaining - above, out, cap, sh.cnt[0]);
        remaining = 0;
        return true;
    }
    remaining -= above;
    prefix |= (uint32_t)bin << SHIFT;
    pmask |= dmask << SHIFT;
    return true;
}

// Levels 1 and 2 (bits [19:9], then [8:0]) over m elements restricted to
// (key & pmask) == prefix; emits the `remaining` best of them at
// out[sh.cnt[0] ...] (slots below cap).  Both level histograms must be clear
// (Scratch::clear_levels before an earlier barrier).  All threads.  Rows
// left equal on all 32 bits are taken in element order, so two calls over
// the same elements with budgets a <= b take nested sets.
template <int T, class Src, int U = 8>
__device__ __forceinline__ void finish_levels(const Src &src, int m, uint32_t prefix, uint32_t pmask, uint32_t remaining,
                              int32_t *out, int cap, Scratch<T> &sh)
{
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if (remaining == 0) return;
    if (m <= 64) { // the callers' barrier has published the list and the output count
        if (tid < 64) rank_take(src, m, nullptr, prefix, pmask, remaining, out, cap, sh.cnt[0]);
        return;
    }
    if (!digit_level<T, Src, U, 9, 2048>(src, m, prefix, pmask, remaining, out, cap, sh.hist, sh)) return;
    if (remaining == 0) return;
    if (!digit_level<T, Src, U, 0, 512>(src, m, prefix, pmask, remaining, out, cap, sh.hist2, sh)) return;
    if (remaining == 0) return;
    // All 32 bits resolved: the survivors share one key.  Take the first
    // `remaining` of them in element order (rank by a block-wide count).
    __syncthreads(); // every thread has read sh.res before wtot is reused
    uint32_t base = 0;
    for (int i0 = 0; i0 < m && base < remaining; i0 += T) {
        const int i = i0 + tid;
        const bool tie = i < m && src.key(i) == prefix;
        const uint64_t tm = __ballot(tie);
        if (lane == 0) sh.wtot[wv] = (uint32_t)__popcll(tm);
        __syncthreads();
        uint32_t before = base, total = 0;
        for (int w2 = 0; w2 < T / 64; ++w2) {
            const uint32_t v = sh.wtot[w2];
            before += w2 < wv ? v : 0u;
            total += v;
        }
        const bool take[1] = {tie && before + (uint32_t)__popcll(tm & lanes_below()) < remaining};
        __syncthreads();
        wave_append<1>(take, &sh.cnt[0], cap, [&](int, int slot) { out[slot] = src.out(i); });
        base += total;
    }
}

// ---------------------------------------------------------------------------
// One workgroup per query.  HIST: the scoring kernel counted the first digit
// into the global histogram and recorded n; otherwise both are found here.
//   kSmall  (max_n <= kCandCap): keys, output ids, histogram and n load once,
//           all at the start, and everything after that runs in LDS;
//   kCached (no histogram, max_n <= kKeyCache): the counting pass keeps the
//           keys in LDS for the emission pass;
//   kStream (longer rows): two passes over the row (one with a histogram),
//           a smaller LDS footprint so that two workgroups share a CU;
//   kSmall2 (no histogram, max_n <= 2 * kCandCap): kSmall with twice the
//           keys per thread and a tie list as long as the row, for a few
//           queries of up to 16384 rows (about 150 KiB of LDS: one
//           workgroup per CU, which a few queries leave idle anyway).
// ---------------------------------------------------------------------------
enum { kSmall = 0, kCached = 1, kStream = 2, kSmall2 = 3 };
constexpr int kStreamCap = 4096; // tied rows kept in LDS by the streaming mode

// A few queries of 8193..16384 rows are selected by kSmall2, from keys the
// selection counts itself (the scoring kernel then counts nothing).
constexpr bool use_small2(int64_t Q, int64_t max_n) { return max_n > kCandCap && max_n <= 2 * kCandCap && Q <= 64; }

// Keys and output ids of elements e * T + tid (e < E) of a row of at most mx
// elements (zero past mx).  The map and the row are branched on once, not
// per element, and indices are clamped into the row, so every load of a
// phase is in flight at once: one round trip for the map, one for the keys
// and ids.  Map entries past the row's count may be -1; they read element 0,
// whose key is never used for them.
template <int E>
__device__ __forceinline__ void load_small(const SelRow &r, int q, int mx, uint32_t (&kk)[E], int32_t (&id)[E])
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        kk[e] = 0u;
        id[e] = 0;
    }
    if (mx <= 0) return;
    int64_t j[E];
#pragma unroll
    for (int e = 0; e < E; ++e) j[e] = min(e * NT + tid, mx - 1);
    if (r.gmap) {
        const int32_t *g = r.gmap + (int64_t)q * r.gld;
        int32_t v[E];
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = g[j[e]];
#pragma unroll
        for (int e = 0; e < E; ++e) j[e] = v[e] < 0 ? 0 : (v[e] < r.ld ? v[e] : r.ld - 1);
    }
    const float *S = r.S + (int64_t)q * r.ld;
    float s[E];
#pragma unroll
    for (int e = 0; e < E; ++e) s[e] = S[j[e]];
    if (r.omap) {
        const int32_t *o = r.omap + (int64_t)q * r.old;
#pragma unroll
        for (int e = 0; e < E; ++e) id[e] = o[min(e * NT + tid, mx - 1)];
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) id[e] = e * NT + tid;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const bool live = e * NT + tid < mx;
        kk[e] = live ? score_key(s[e]) : 0u;
        id[e] = live ? id[e] : 0;
    }
}

template <int MODE>
constexpr int select_cap()
{
    return MODE == kStream ? kStreamCap : (MODE == kSmall2 ? 2 * kCandCap : kCandCap);
}

// select_query on LDS the caller provides: the digit histogram h0
// [kHistBins], the tie list ck / ci [select_cap<MODE>()] and, in the cached
// mode, the key cache [kKeyCache].
template <bool HIST, int MODE>
__device__ __forceinline__ void select_query_in(const SelCall &c, const SelWorkspace &ws, Scratch<NT> &sh,
                                                uint32_t *h0, uint32_t *ck, int32_t *ci, uint32_t *cache)
{
    constexpr int CAP = select_cap<MODE>();
    constexpr int KB = kB;
    const int tid = threadIdx.x;
    const int q = blockIdx.x;
    const int32_t *hq = ws.hist + (int64_t)q * kHistStride;
    int32_t *out = c.idx + (int64_t)q * c.k;
    if (tid == 0) {
        sh.cnt[0] = 0;
        sh.cnt[1] = 0;
    }
    sh.clear_levels();
    int K = 0;
    if constexpr (MODE == kSmall || MODE == kSmall2) {
        constexpr int E = CAP / NT;
        const int mx = (int)c.max_n;
        uint32_t kk[E];
        int32_t id[E];
        load_small<E>(c.row, q, mx, kk, id);
        HistRegs<NT> hr;
        int n;
        if constexpr (HIST) {
            hr.load(hq);
            n = clamp_n(hq[kSlotN], mx);
        } else {
            n = query_n(c, q);
        }
        K = min(n, c.k);
        if (K > 0 && K == n) {
            // the budget covers the whole row: every element is taken
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (e * NT + tid < n) out[e * NT + tid] = id[e];
        } else if (K > 0) {
            if constexpr (HIST) {
                hr.store(h0);
            } else {
                // The keys of the row move to (key - min) << s, s as large as
                // the row's key range allows: a strictly increasing map, so
                // the selection and its ties are those of the raw keys, but
                // the first digit now splits the row's own range 4096 ways
                // (rows of similar scores otherwise pile into a few bins of
                // the raw top 12 bits: contended counts, long tie lists).
                uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (e * NT + tid < n) {
                        lo = min(lo, kk[e]);
                        hi = max(hi, kk[e]);
                    }
                wave_min_max(lo, hi);
                if ((tid & 63) == 0) {
                    sh.wlo[tid >> 6] = lo;
                    sh.whi[tid >> 6] = hi;
                }
                for (int j = tid; j < kHistBins; j += NT) h0[j] = 0;
                __syncthreads();
#pragma unroll
                for (int w2 = 0; w2 < NT / 64; ++w2) {
                    lo = min(lo, sh.wlo[w2]);
                    hi = max(hi, sh.whi[w2]);
                }
                const int bits = 32 - __clz(hi - lo);               // bits of the key range
                const int shl = kDigit0Shift - max(bits - 12, 0); // left shift, 0..20
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    if (e * NT + tid < n) {
                        kk[e] = (kk[e] - lo) << shl;
                        atomicAdd(&h0[kk[e] >> kDigit0Shift], 1u);
                    }
                }
            }
            __syncthreads();
            const uint32_t rem[1] = {(uint32_t)K};
            find_bins<NT, kHistBins, 1>(h0, rem, sh);
            const int bin = sh.res[0];
            const int above = sh.res[1];
            if (bin >= 0) {
                bool up[E], tie[E];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const bool ok = e * NT + tid < n;
                    const int dg = (int)(kk[e] >> kDigit0Shift);
                    up[e] = ok && dg > bin;
                    tie[e] = ok && dg == bin;
                }
                wave_append<E>(up, &sh.cnt[0], c.k, [&](int u, int slot) { out[slot] = id[u]; });
                wave_append<E>(tie, &sh.cnt[1], CAP, [&](int u, int slot) {
                    ck[slot] = kk[u];
                    ci[slot] = id[u];
                });
                __syncthreads();
                finish_levels<NT>(CandLds{ck, ci}, min(sh.cnt[1], CAP), (uint32_t)bin << kDigit0Shift,
                                  0xFFFFFFFFu << kDigit0Shift, (uint32_t)(K - above), out, c.k, sh);
            }
        }
    } else {
        int n;
        if constexpr (HIST) {
            n = clamp_n(hq[kSlotN], c.max_n);
        } else {
            n = query_n(c, q);
        }
        K = min(n, c.k);
        const bool cached = MODE == kCached && n <= kKeyCache;
        constexpr int64_t ROUND = (int64_t)NT * KB * 4;
        if (K > 0 && K == n) {
            for (int i = tid; i < n; i += NT) out[i] = out_id(c.row, q, i); // the budget covers the whole row
        } else if (K > 0) {
            if constexpr (HIST) {
                HistRegs<NT> hr;
                hr.load(hq);
                hr.store(h0);
                __syncthreads();
                const uint32_t rem[1] = {(uint32_t)K};
                find_bins<NT, kHistBins, 1>(h0, rem, sh);
            } else {
                for (int j = tid; j < kHistBins; j += NT) h0[j] = 0;
                __syncthreads();
                for (int64_t r0 = 0; r0 < n; r0 += ROUND) {
                    uint32_t kk[KB][4];
#pragma unroll
                    for (int b = 0; b < KB; ++b) keys4(c.row, q, r0 + 4 * ((int64_t)b * NT + tid), n, kk[b]);
#pragma unroll
                    for (int b = 0; b < KB; ++b)
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const int64_t i = r0 + 4 * ((int64_t)b * NT + tid) + t;
                            if (i < n) {
                                atomicAdd(&h0[kk[b][t] >> kDigit0Shift], 1u);
                                if constexpr (MODE == kCached)
                                    if (cached) cache[i] = kk[b][t];
                            }
                        }
                }
                __syncthreads();
                const uint32_t rem[1] = {(uint32_t)K};
                find_bins<NT, kHistBins, 1>(h0, rem, sh);
            }
            const int bin = sh.res[0];
            const int above = sh.res[1];
            if (bin >= 0) {
                // one pass over the row: emit above, keep ties
                for (int64_t r0 = 0; r0 < n; r0 += ROUND) {
                    uint32_t kk[KB][4];
#pragma unroll
                    for (int b = 0; b < KB; ++b) {
                        const int64_t i = r0 + 4 * ((int64_t)b * NT + tid);
                        if (cached) {
#pragma unroll
                            for (int t = 0; t < 4; ++t) kk[b][t] = i + t < n ? cache[i + t] : 0u;
                        } else {
                            keys4(c.row, q, i, n, kk[b]);
                        }
                    }
#pragma unroll
                    for (int b = 0; b < KB; ++b) {
                        const int64_t i4 = r0 + 4 * ((int64_t)b * NT + tid);
                        bool up[4], tie[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const int dg = (int)(kk[b][t] >> kDigit0Shift);
                            const bool ok = i4 + t < n;
                            up[t] = ok && dg > bin;
                            tie[t] = ok && dg == bin;
                        }
                        wave_append<4>(up, &sh.cnt[0], c.k, [&](int t, int slot) { out[slot] = out_id(c.row, q, i4 + t); });
                        wave_append<4>(tie, &sh.cnt[1], CAP, [&](int t, int slot) {
                            ck[slot] = kk[b][t];
                            ci[slot] = out_id(c.row, q, i4 + t);
                        });
                    }
                }
                __syncthreads();
                const int nc = sh.cnt[1];
                const uint32_t prefix = (uint32_t)bin << kDigit0Shift;
                const uint32_t pmask = 0xFFFFFFFFu << kDigit0Shift;
                const uint32_t need = (uint32_t)(K - above);
                // batch depth of the level passes: 2 in the streaming mode,
                // which runs in 64 registers
                constexpr int UB = MODE == kStream ? 2 : 8;
                if (nc <= CAP) {
                    finish_levels<NT, CandLds, UB>(CandLds{ck, ci}, nc, prefix, pmask, need, out, c.k, sh);
                } else if (cached) {
                    finish_levels<NT, CacheLds, UB>(CacheLds{cache, c.row, q}, n, prefix, pmask, need, out, c.k,
                                                    sh);
                } else {
                    finish_levels<NT, RowGlobal, UB>(RowGlobal{c.row, q}, n, prefix, pmask, need, out, c.k, sh);
                }
            }
        }
    }
    for (int i = K + tid; i < c.k; i += NT) out[i] = -1;
    if (tid == 0) c.count[q] = K;
}

template <bool HIST, int MODE>
__device__ __forceinline__ void select_query(const SelCall &c, const SelWorkspace &ws)
{
    __shared__ Scratch<NT> sh;
    __shared__ uint32_t h0[kHistBins];
    __shared__ uint32_t ck[select_cap<MODE>()];
    __shared__ int32_t ci[select_cap<MODE>()];
    __shared__ uint32_t cache[MODE == kCached ? kKeyCache : 1];
    select_query_in<HIST, MODE>(c, ws, sh, h0, ck, ci, cache);
}

template <bool HIST, int MODE>
__global__ __launch_bounds__(NT) void k_select(SelCall c, SelWorkspace ws)
{
    select_query<HIST, MODE>(c, ws);
}

// Streaming mode: its LDS footprint lets two 1024-thread workgroups share a
// CU once the registers fit 8 waves per SIMD.
template <bool HIST>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(8))) void k_select_stream(SelCall c,
                                                                                            SelWorkspace ws)
{
    select_query<HIST, kStream>(c, ws);
}

template <bool HIST>
hipError_t launch_k_select(const SelCall &c, const SelWorkspace &ws, hipStream_t s)
{
    if (c.max_n <= kCandCap) {
        hipLaunchKernelGGL((k_select<HIST, kSmall>), dim3(c.Q), dim3(NT), 0, s, c, ws);
        return hipGetLastError();
    }
    if constexpr (!HIST) {
        if (use_small2(c.Q, c.max_n)) {
            hipLaunchKernelGGL((k_select<HIST, kSmall2>), dim3(c.Q), dim3(NT), 0, s, c, ws);
            return hipGetLastError();
        }
        if (c.max_n <= kKeyCache) {
            hipLaunchKernelGGL((k_select<HIST, kCached>), dim3(c.Q), dim3(NT), 0, s, c, ws);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((k_select_stream<HIST>), dim3(c.Q), dim3(NT), 0, s, c, ws);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Few queries, long rows: many workgroups per query stream the row once.
// Each emits its rows above the threshold digit(s) and appends the rows on
// them to the tie lists.  With a nested selection (k_inner > 0) the inner
// threshold digit is found from the same histogram and served in the same
// pass; its ties share the outer list when both digits coincide.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kFilterThreads) void k_filter(SelCall c, SelWorkspace ws)
{
    constexpr int T = kFilterThreads;
    __shared__ Scratch<T> sh;
    __shared__ uint32_t h0[kHistBins];
    __shared__ int s_cnt[4];
    __shared__ int s_base[4];
    const int tid = threadIdx.x;
    const int q = blockIdx.y;
    const int64_t i0 = (int64_t)blockIdx.x * kFilterChunk;
    int32_t *hq = ws.hist + (int64_t)q * kHistStride;
    // Loaded up front, together: this workgroup's keys (bounded by max_n,
    // masked by n below), the histogram and n.
    uint32_t kk[kB][4];
#pragma unroll
    for (int b = 0; b < kB; ++b) keys4(c.row, q, i0 + 4 * ((int64_t)b * T + tid), c.max_n, kk[b]);
    HistRegs<T> hr;
    hr.load(hq);
    const int n = clamp_n(hq[kSlotN], c.max_n);
    const int K = min(n, c.k);
    const int Ki = c.k_inner > 0 ? min(n, c.k_inner) : 0;
    if (K == 0 || i0 >= n) return;
    if (tid < 4) s_cnt[tid] = 0;
    hr.store(h0);
    __syncthreads();
    const uint32_t rem[2] = {(uint32_t)K, (uint32_t)(Ki > 0 ? Ki : K)};
    find_bins<T, kHistBins, 2>(h0, rem, sh);
    const int bin = sh.res[0];
    const int bin_i = Ki > 0 ? sh.res[2] : -1;
    if (blockIdx.x == 0 && tid == 0) { // every workgroup finds the same digits; the final kernel reads them here
        hq[kSlotBins] = (int32_t)(((uint32_t)sh.res[0] & 0xFFFFu) | ((uint32_t)sh.res[2] << 16));
        hq[kSlotAboveO] = sh.res[1];
        hq[kSlotAboveI] = sh.res[3];
    }
    // a histogram that does not hold exactly n rows (inconsistent counts)
    // leaves this workgroup's rows unsorted, and the final kernel redoes the query
    if (sh.wtot[0] + sh.wtot[1] + sh.wtot[2] + sh.wtot[3] != (uint32_t)n) return;
    if (bin < 0 || (Ki > 0 && bin_i < 0)) return;
    const bool inner = Ki > 0;
    const bool sep = inner && bin_i != bin; // inner ties need a list of their own
    int nup = 0, ntie = 0, nupi = 0, ntiei = 0;
#pragma unroll
    for (int b = 0; b < kB; ++b)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int64_t i = i0 + 4 * ((int64_t)b * T + tid) + t;
            const int dg = (int)(kk[b][t] >> kDigit0Shift);
            if (i < n) {
                nup += dg > bin;
                ntie += dg == bin;
                if (inner) {
                    nupi += dg > bin_i;
                    ntiei += sep && dg == bin_i;
                }
            }
        }
    // this thread's offsets in the workgroup's four runs: an exclusive wave
    // scan plus one LDS atomic per wave and run
    const int cnts[4] = {nup, ntie, nupi, ntiei};
    int loc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t incl = wave_incl_scan((uint32_t)cnts[j]);
        const int wt = __builtin_amdgcn_readlane((int)incl, 63);
        int wb = 0;
        if (wt && (tid & 63) == 0) wb = atomicAdd(&s_cnt[j], wt);
        wb = __builtin_amdgcn_readfirstlane(wb);
        loc[j] = wb + (int)incl - cnts[j];
    }
    __syncthreads();
    if (tid < 4) {
        const int slot = tid == 0 ? kSlotUpO : tid == 1 ? kSlotTieO : tid == 2 ? kSlotUpI : kSlotTieI;
        const int v = s_cnt[tid];
        s_base[tid] = v ? atomicAdd(&hq[slot], v) : 0;
    }
    __syncthreads();
    int pu = s_base[0] + loc[0], pt = s_base[1] + loc[1], pui = s_base[2] + loc[2], pti = s_base[3] + loc[3];
    int32_t *out = c.idx + (int64_t)q * c.k;
    int32_t *outi = inner ? c.idx_inner + (int64_t)q * c.k_inner : nullptr;
    uint2 *cand = ws.cand + (int64_t)q * ws.cap;
    uint2 *cand2 = ws.cand2 + (int64_t)q * ws.cap;
#pragma unroll
    for (int b = 0; b < kB; ++b)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int64_t i = i0 + 4 * ((int64_t)b * T + tid) + t;
            if (i < n) {
                const int dg = (int)(kk[b][t] >> kDigit0Shift);
                if (dg > bin) {
                    if (pu < c.k) out[pu] = out_id(c.row, q, i);
                    ++pu;
                } else if (dg == bin) {
                    if (pt < ws.cap) cand[pt] = make_uint2(kk[b][t], (uint32_t)i);
                    ++pt;
                }
                if (inner) {
                    if (dg > bin_i) {
                        if (pui < c.k_inner) outi[pui] = out_id(c.row, q, i);
                        ++pui;
                    } else if (sep && dg == bin_i) {
                        if (pti < ws.cap) cand2[pti] = make_uint2(kk[b][t], (uint32_t)i);
                        ++pti;
                    }
                }
            }
        }
    if (tid == 0) // this workgroup's rows are sorted
        atomicAdd(&hq[kSlotDone], (int)((int64_t)n - i0 < kFilterChunk ? (int64_t)n - i0 : kFilterChunk));
}

// What a call added to the query's entry of the workspace's zeroed region:
// the histogram, the row total and the published digits (the scoring
// kernel's first workgroup zeroes the other counters itself).  The final
// kernel's outer workgroup, which no other reader of them outlives.
__device__ __forceinline__ void clear_sync(int32_t *hq)
{
    const int tid = threadIdx.x;
    for (int j = tid; j < kHistBins; j += NT) hq[j] = 0;
    if (tid == 0) {
        hq[kSlotTotal] = 0;
        hq[kSlotResult] = 0;
        hq[kSlotResult + 1] = 0;
    }
}

// The whole selection of query blockIdx.x from its scores (the streaming
// one-workgroup mode), then the nested one over the outer winners: the
// final kernel's fallback when the fused filter pass did not complete.
__device__ __forceinline__ void final_from_scores(const SelCall &c, const SelWorkspace &ws, Scratch<NT> &sh,
                                                  uint32_t *h0, uint32_t *ck, int32_t *ci)
{
    SelCall oc = c;
    oc.k_inner = 0;
    oc.idx_inner = nullptr;
    oc.count_inner = nullptr;
    select_query_in<false, kStream>(oc, ws, sh, h0, ck, ci, nullptr);
    if (c.k_inner <= 0) return;
    __syncthreads(); // the outer winners and their count are visible to the whole workgroup
    SelCall ic = oc;
    ic.row = SelRow{c.row.S, c.row.ld, c.idx, c.k, c.idx, c.k};
    ic.src_mode = kSrcCount;
    ic.cnt = c.count;
    ic.cnt_cap = c.k;
    ic.k = c.k_inner;
    ic.max_n = std::min<int64_t>(c.k, c.max_n);
    ic.idx = c.idx_inner;
    ic.count = c.count_inner;
    select_query_in<false, kStream>(ic, ws, sh, h0, ck, ci, nullptr);
}

// The remaining digits among the tied rows: blockIdx.y = 0 for the outer
// selection, 1 for the nested one, one workgroup per query each.
__global__ __launch_bounds__(NT) void k_final(SelCall c, SelWorkspace ws)
{
    __shared__ Scratch<NT> sh;
    __shared__ uint32_t ck[kCandCap];
    __shared__ int32_t ci[kCandCap];
    constexpr int E = kCandCap / NT;
    const int tid = threadIdx.x;
    const int q = blockIdx.x;
    const bool inner = blockIdx.y == 1;
    int32_t *hq = ws.hist + (int64_t)q * kHistStride;
    const int kout = inner ? c.k_inner : c.k;
    int32_t *out = (inner ? c.idx_inner : c.idx) + (int64_t)q * kout;
    sh.clear_levels();
    // Loaded up front: the threshold digits the filter found, the counters,
    // and the head of this part's tie list (the nested part's list is the
    // likely one; the outer list is read later only when the two threshold
    // digits coincide).
    const int lim = (int)(ws.cap < kCandCap ? ws.cap : kCandCap);
    const uint2 *list = (inner ? ws.cand2 : ws.cand) + (int64_t)q * ws.cap;
    uint2 p[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = e * NT + tid;
        p[e] = i < lim ? list[i] : make_uint2(0u, 0u);
    }
    const int n = clamp_n(hq[kSlotN], c.max_n);
    const int tie_o = hq[kSlotTieO];
    const int tie_i = hq[kSlotTieI];
    const int bins = hq[kSlotBins];
    const int above_o = hq[kSlotAboveO];
    const int above_i = hq[kSlotAboveI];
    if (hq[kSlotDone] != n) {
        // The filter pass did not sort every row: a workgroup of a fused pass
        // gave up waiting for the others (the grid was not all resident at
        // once), or the histogram was inconsistent.  The selection runs again
        // from the scores alone, the nested one over the outer winners.
        static_assert(kHistBins + kStreamCap <= kCandCap && kStreamCap <= kCandCap, "fallback LDS");
        if (!inner) {
            final_from_scores(c, ws, sh, ck, ck + kHistBins, ci);
            clear_sync(hq);
        }
        return;
    }
    const int K = min(n, c.k);
    const int Kp = inner ? min(n, c.k_inner) : K;
    if (Kp > 0) {
        const int bin_o = (int)(int16_t)(bins & 0xFFFF);
        const int bin = inner ? (int)(int16_t)(bins >> 16) : bin_o;
        const int above = inner ? above_i : above_o;
        if (bin >= 0 && bin_o >= 0) {
            const bool shared_list = inner && bin == bin_o;
            const int nc = inner && !shared_list ? tie_i : tie_o;
            if (shared_list) {
                const uint2 *lo = ws.cand + (int64_t)q * ws.cap;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int i = e * NT + tid;
                    p[e] = i < lim ? lo[i] : make_uint2(0u, 0u);
                }
            }
            if (tid == 0) sh.cnt[0] = above;
            const uint32_t prefix = (uint32_t)bin << kDigit0Shift;
            const uint32_t pmask = 0xFFFFFFFFu << kDigit0Shift;
            const uint32_t need = (uint32_t)(Kp - above);
            if (nc <= lim) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int i = e * NT + tid;
                    if (i < nc) {
                        ck[i] = p[e].x;
                        ci[i] = out_id(c.row, q, (int64_t)p[e].y);
                    }
                }
                __syncthreads();
                finish_levels<NT>(CandLds{ck, ci}, nc, prefix, pmask, need, out, kout, sh);
            } else if (nc <= ws.cap) {
                // every tie is in the global list: rank it instead of the row
                const uint2 *lst = (inner && !shared_list ? ws.cand2 : ws.cand) + (int64_t)q * ws.cap;
                __syncthreads(); // the level histograms' clear and the output count
                finish_levels<NT>(CandGlobal{lst, c.row, q}, nc, prefix, pmask, need, out, kout, sh);
            } else {
                __syncthreads();
                finish_levels<NT>(RowGlobal{c.row, q}, n, prefix, pmask, need, out, kout, sh);
            }
        }
    }
    for (int i = Kp + tid; i < kout; i += NT) out[i] = -1;
    if (tid == 0) (inner ? c.count_inner : c.count)[q] = Kp;
    if (!inner) clear_sync(hq);
}

// Clears the per-query histograms and slots before a scoring kernel
// accumulates into them.
__global__ __launch_bounds__(256) void k_hist_clear(int32_t *hist, int64_t words)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (int64_t)gridDim.x * 256) hist[i] = 0;
}

bool use_filter(int64_t Q, int64_t max_n) { return max_n > kKeyCache && Q <= kSyncQueries; }

int64_t cand_cap(int64_t Q, int64_t max_n) { return use_filter(Q, max_n) ? std::min<int64_t>(max_n, 65536) : 0; }

} // namespace

bool selection_wants_counts(int64_t Q, int64_t max_n) { return max_n > kCandCap && !use_small2(Q, max_n); }

size_t sel_workspace_bytes(int64_t Q, int64_t max_n)
{
    size_t b = (size_t)Q * kHistStride * 4;
    b = (b + 255) & ~(size_t)255;
    return b + 2 * (size_t)Q * cand_cap(Q, max_n) * 8;
}

SelWorkspace sel_workspace_carve(void *base, int64_t Q, int64_t max_n, int32_t *sync)
{
    SelWorkspace w;
    w.hist = use_filter(Q, max_n) ? sync : (int32_t *)base;
    size_t off = ((size_t)Q * kHistStride * 4 + 255) & ~(size_t)255;
    w.cap = cand_cap(Q, max_n);
    w.cand = (uint2 *)((uint8_t *)base + off);
    w.cand2 = w.cand + Q * w.cap;
    return w;
}

hipError_t launch_hist_clear(const SelWorkspace &ws, int64_t Q, hipStream_t s)
{
    const int64_t words = Q * kHistStride;
    const int64_t blocks = std::min<int64_t>((words + 255) / 256, 2048);
    hipLaunchKernelGGL(k_hist_clear, dim3((unsigned)blocks), dim3(256), 0, s, ws.hist, words);
    return hipGetLastError();
}

bool selection_filters(int64_t Q, int64_t max_n) { return use_filter(Q, max_n); }

hipError_t launch_select(const SelCall &c, const SelWorkspace &ws, bool have_hist, hipStream_t s, bool filtered)
{
    if (c.Q <= 0) return hipSuccess;
    if (have_hist && use_filter(c.Q, c.max_n)) {
        if (!filtered) { // else the scoring kernel ran the filter pass
            const int64_t chunks = (c.max_n + kFilterChunk - 1) / kFilterChunk;
            hipLaunchKernelGGL(k_filter, dim3((unsigned)chunks, c.Q), dim3(kFilterThreads), 0, s, c, ws);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(k_final, dim3(c.Q, c.k_inner > 0 ? 2 : 1), dim3(NT), 0, s, c, ws);
        return hipGetLastError();
    }
    hipError_t e = have_hist ? launch_k_select<true>(c, ws, s) : launch_k_select<false>(c, ws, s);
    if (e != hipSuccess || c.k_inner <= 0) return e;
    // Nested selection among the outer winners (a subset by construction).
    SelCall ic = c;
    ic.row = SelRow{c.row.S, c.row.ld, c.idx, c.k, c.idx, c.k};
    ic.src_mode = kSrcCount;
    ic.cnt = c.count;
    ic.cnt_cap = c.k;
    ic.k = c.k_inner;
    ic.max_n = std::min<int64_t>(c.k, c.max_n);
    ic.idx = c.idx_inner;
    ic.count = c.count_inner;
    ic.k_inner = 0;
    ic.idx_inner = nullptr;
    ic.count_inner = nullptr;
    return launch_k_select<false>(ic, ws, s);
}

} // namespace li

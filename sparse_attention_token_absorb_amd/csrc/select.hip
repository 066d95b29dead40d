// Per-query top-k selection (gfx950).
//
// LatentIndex (paperlayer.ai summary of arXiv:2610.04635), §3.1/§4.1: every
// layer picks its own top-k rows (k = 2048), capped by the valid prefix
// (§C.4); the HS anchor picks its top-M candidates and its own top-k inside
// them (§3.2, §C.4).
//
// Scores become order-preserving uint32 keys, selected by radix digits of
// 12, 11 and 9 bits (most significant first).  The scoring kernels already
// count the first digit (key >> 20) into a per-query 4096-bin histogram as
// they write the scores, so the threshold bin is known before the rows are
// read again.  One pass over each row then emits the rows above the
// threshold digit and compacts the rows on it; the last two digits are
// resolved among those few in LDS.
//   * Few queries with long rows (decode at 8K-128K): the pass is spread
//     over many workgroups per query (k_filter), and one workgroup per
//     query finishes (k_final).
//   * Many queries or short rows (prefill, HS followers, the anchor's nested
//     selection): one 1024-thread workgroup per query does it all (k_select).
// Rows are read 16 bytes per lane, several loads in flight per thread (the
// scores were written by other XCDs, so every load misses the local L2).
// Emission uses wavefront ballots (one LDS atomic per wave, mbcnt offsets).
// Rows whose key equals the final threshold key are taken in arbitrary
// order, as many as the budget needs: equal scores are interchangeable.
#include "li_internal.hpp"

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
    const int64_t j = r.gmap ? (int64_t)r.gmap[(int64_t)q * r.gld + i] : i;
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

__device__ __forceinline__ int query_n(const SelCall &c, int q)
{
    int n;
    if (c.src_mode == kSrcCausal) {
        n = valid_rows(c.qpos[q], c.seq_lens[c.qseq[q]]);
    } else {
        n = c.cnt[q] < c.cnt_cap ? c.cnt[q] : c.cnt_cap;
        n = n > 0 ? n : 0;
    }
    return n < c.max_n ? n : (int)c.max_n; // the caller's bound sizes every buffer
}

__device__ __forceinline__ uint64_t lanes_below() { return (1ull << (threadIdx.x & 63)) - 1ull; }

template <int T>
struct Scratch {
    uint32_t hist[2048];
    uint32_t wtot[T / 64];
    int res[2];
    int cnt[4];
};

// Block-wide search on an LDS histogram of nbins bins: the bin b holding
// the `remaining`-th largest element and `above` = elements in bins > b.
// sh.res[0] = b (-1 if remaining exceeds the total), sh.res[1] = above.
template <int T>
__device__ void find_bin(const uint32_t *h, int nbins, uint32_t remaining, Scratch<T> &sh)
{
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int per = (nbins + T - 1) / T;
    uint32_t sum = 0;
    for (int j = 0; j < per; ++j) {
        const int bb = tid * per + j;
        if (bb < nbins) sum += h[bb];
    }
    uint32_t suf = sum; // suffix sum within the wave: lanes >= lane
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_down(suf, off);
        if (lane + off < 64) suf += v;
    }
    if (lane == 0) sh.wtot[wv] = suf;
    if (tid == 0) sh.res[0] = -1;
    __syncthreads();
    uint32_t later = 0;
    for (int w2 = wv + 1; w2 < T / 64; ++w2) later += sh.wtot[w2];
    const uint32_t incl = suf + later;
    const uint32_t excl = incl - sum;
    if (excl < remaining && incl >= remaining) {
        uint32_t acc = excl;
        for (int j = per - 1; j >= 0; --j) {
            const int bb = tid * per + j;
            if (bb >= nbins) continue;
            if (acc + h[bb] >= remaining) {
                sh.res[0] = bb;
                sh.res[1] = (int)acc;
                break;
            }
            acc += h[bb];
        }
    }
    __syncthreads();
}

// Lanes with e set append `val` at out[*cnt ...] (one LDS atomic per wave).
// Whole waves must reach it.
__device__ __forceinline__ void emit(bool e, int32_t val, int32_t *out, int *cnt)
{
    const uint64_t m = __ballot(e);
    if (m == 0ull) return;
    int base = 0;
    if ((threadIdx.x & 63) == 0) base = atomicAdd(cnt, __popcll(m));
    base = __shfl(base, 0);
    if (e) out[base + __popcll(m & lanes_below())] = val;
}

// Digits below the first: bits [19:9] then [8:0].
__device__ __forceinline__ int lvl_shift(int l) { return l == 1 ? 9 : 0; }
__device__ __forceinline__ int lvl_bins(int l) { return l == 1 ? 2048 : 512; }

// Element sources for the in-block levels: key(i), id(i).
struct CandLds {
    const uint32_t *k;
    const int32_t *d;
    __device__ uint32_t key(int i) const { return k[i]; }
    __device__ int64_t id(int i) const { return d[i]; }
};
struct CacheLds {
    const uint32_t *k;
    __device__ uint32_t key(int i) const { return k[i]; }
    __device__ int64_t id(int i) const { return i; }
};
struct RowGlobal {
    SelRow r;
    int q;
    __device__ uint32_t key(int i) const { return key_at(r, q, i); }
    __device__ int64_t id(int i) const { return i; }
};

// Levels 1 and 2 over m elements restricted to (key & pmask) == prefix;
// emits the `remaining` best of them at out[sh.cnt[0] ...].  All threads.
template <int T, class Src>
__device__ void finish_levels(const Src &src, int m, uint32_t prefix, uint32_t pmask, uint32_t remaining,
                              int32_t *out, const SelRow &row, int q, Scratch<T> &sh)
{
    const int tid = threadIdx.x, lane = tid & 63;
    const int wbase = tid - lane;
    int level = 1;
    for (; level < 3 && remaining > 0; ++level) {
        const int shift = lvl_shift(level);
        const int nb = lvl_bins(level);
        const uint32_t dmask = (uint32_t)nb - 1u;
        for (int j = tid; j < nb; j += T) sh.hist[j] = 0;
        __syncthreads();
        for (int i = tid; i < m; i += T) {
            const uint32_t key = src.key(i);
            if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & dmask], 1u);
        }
        __syncthreads();
        find_bin<T>(sh.hist, nb, remaining, sh);
        const int bin = sh.res[0];
        const uint32_t above = (uint32_t)sh.res[1];
        if (bin < 0) break; // inconsistent counts: nothing sensible to emit
        for (int i0 = wbase; i0 < m; i0 += T) {
            const int i = i0 + lane;
            bool e = false;
            if (i < m) {
                const uint32_t key = src.key(i);
                e = (key & pmask) == prefix && ((key >> shift) & dmask) > (uint32_t)bin;
            }
            emit(e, e ? out_id(row, q, src.id(i)) : 0, out, &sh.cnt[0]);
        }
        remaining -= above;
        prefix |= (uint32_t)bin << shift;
        pmask |= dmask << shift;
        __syncthreads();
    }
    if (remaining > 0 && level == 3) {
        // all 32 bits resolved: the survivors share one key
        if (tid == 0) sh.cnt[2] = 0;
        __syncthreads();
        for (int i0 = wbase; i0 < m; i0 += T) {
            const int i = i0 + lane;
            const bool tie = i < m && src.key(i) == prefix;
            const uint64_t tm = __ballot(tie);
            if (tm == 0ull) continue;
            int base = 0;
            if (lane == 0) base = atomicAdd(&sh.cnt[2], __popcll(tm));
            base = __shfl(base, 0);
            const bool take = tie && (uint32_t)(base + __popcll(tm & lanes_below())) < remaining;
            emit(take, take ? out_id(row, q, src.id(i)) : 0, out, &sh.cnt[0]);
        }
    }
    __syncthreads();
}

// Threshold bin of the first digit from the query's global histogram.
template <int T>
__device__ void threshold_from_hist(const int32_t *g, uint32_t *h0, int K, Scratch<T> &sh)
{
    constexpr int PER = kHistBins / T;
    uint32_t v[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) v[e] = (uint32_t)g[e * T + threadIdx.x];
#pragma unroll
    for (int e = 0; e < PER; ++e) h0[e * T + threadIdx.x] = v[e];
    __syncthreads();
    find_bin<T>(h0, kHistBins, (uint32_t)K, sh);
}

// ---------------------------------------------------------------------------
// One workgroup per query.  HIST: the scoring kernel counted the first digit
// into the global histogram; otherwise it is counted here (rows cached in
// LDS when they fit).
// ---------------------------------------------------------------------------
template <bool HIST>
__global__ __launch_bounds__(NT) void k_select(SelCall c, SelWorkspace ws)
{
    __shared__ Scratch<NT> sh;
    __shared__ uint32_t h0[kHistBins];
    __shared__ uint32_t ck[kCandCap];
    __shared__ int32_t ci[kCandCap];
    __shared__ uint32_t cache[HIST ? 1 : kKeyCache];
    const int tid = threadIdx.x, lane = tid & 63;
    const int q = blockIdx.x;
    const int n = query_n(c, q);
    const int K = min(n, c.k);
    int32_t *out = c.idx + (int64_t)q * c.k;
    const bool cached = !HIST && n <= kKeyCache;
    constexpr int64_t ROUND = (int64_t)NT * kB * 4;
    if (K > 0) {
        if (tid == 0) {
            sh.cnt[0] = 0;
            sh.cnt[1] = 0;
        }
        if constexpr (HIST) {
            threshold_from_hist<NT>(ws.hist + (int64_t)q * kHistStride, h0, K, sh);
        } else {
            for (int j = tid; j < kHistBins; j += NT) h0[j] = 0;
            __syncthreads();
            for (int64_t r0 = 0; r0 < n; r0 += ROUND) {
                uint32_t kk[kB][4];
#pragma unroll
                for (int b = 0; b < kB; ++b) keys4(c.row, q, r0 + 4 * ((int64_t)b * NT + tid), n, kk[b]);
#pragma unroll
                for (int b = 0; b < kB; ++b)
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int64_t i = r0 + 4 * ((int64_t)b * NT + tid) + t;
                        if (i < n) {
                            atomicAdd(&h0[kk[b][t] >> kDigit0Shift], 1u);
                            if (cached) cache[i] = kk[b][t];
                        }
                    }
            }
            __syncthreads();
            find_bin<NT>(h0, kHistBins, (uint32_t)K, sh);
        }
        const int bin = sh.res[0];
        const int above = sh.res[1];
        if (bin >= 0) {
            // one pass over the row: emit above, keep ties
            for (int64_t r0 = 0; r0 < n; r0 += ROUND) {
                uint32_t kk[kB][4];
#pragma unroll
                for (int b = 0; b < kB; ++b) {
                    const int64_t i = r0 + 4 * ((int64_t)b * NT + tid);
                    if (cached) {
#pragma unroll
                        for (int t = 0; t < 4; ++t) kk[b][t] = i + t < n ? cache[i + t] : 0u;
                    } else {
                        keys4(c.row, q, i, n, kk[b]);
                    }
                }
#pragma unroll
                for (int b = 0; b < kB; ++b)
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int64_t i = r0 + 4 * ((int64_t)b * NT + tid) + t;
                        const int dg = (int)(kk[b][t] >> kDigit0Shift);
                        const bool ok = i < n;
                        const bool up = ok && dg > bin;
                        emit(up, up ? out_id(c.row, q, i) : 0, out, &sh.cnt[0]);
                        const bool tie = ok && dg == bin;
                        const uint64_t tm = __ballot(tie);
                        if (tm) {
                            int base = 0;
                            if (lane == 0) base = atomicAdd(&sh.cnt[1], __popcll(tm));
                            base = __shfl(base, 0);
                            const int slot = base + __popcll(tm & lanes_below());
                            if (tie && slot < kCandCap) {
                                ck[slot] = kk[b][t];
                                ci[slot] = (int32_t)i;
                            }
                        }
                    }
            }
            __syncthreads();
            const int nc = sh.cnt[1];
            const uint32_t prefix = (uint32_t)bin << kDigit0Shift;
            const uint32_t pmask = 0xFFFFFFFFu << kDigit0Shift;
            const uint32_t need = (uint32_t)(K - above);
            if (nc <= kCandCap) {
                finish_levels<NT>(CandLds{ck, ci}, nc, prefix, pmask, need, out, c.row, q, sh);
            } else if (cached) {
                finish_levels<NT>(CacheLds{cache}, n, prefix, pmask, need, out, c.row, q, sh);
            } else {
                finish_levels<NT>(RowGlobal{c.row, q}, n, prefix, pmask, need, out, c.row, q, sh);
            }
        }
    }
    for (int i = K + tid; i < c.k; i += NT) out[i] = -1;
    if (tid == 0) c.count[q] = K;
}

// ---------------------------------------------------------------------------
// Few queries, long rows: many workgroups per query stream the row once.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kFilterThreads) void k_filter(SelCall c, SelWorkspace ws)
{
    constexpr int T = kFilterThreads;
    __shared__ Scratch<T> sh;
    __shared__ uint32_t h0[kHistBins];
    __shared__ int s_base[4];
    const int tid = threadIdx.x;
    const int q = blockIdx.y;
    const int n = query_n(c, q);
    const int K = min(n, c.k);
    const int64_t i0 = (int64_t)blockIdx.x * kFilterChunk;
    if (K == 0 || i0 >= n) return;
    int32_t *hist = ws.hist + (int64_t)q * kHistStride;
    threshold_from_hist<T>(hist, h0, K, sh);
    const int bin = sh.res[0];
    if (bin < 0) return;
    if (tid < 4) s_base[tid] = 0;
    uint32_t kk[kB][4];
#pragma unroll
    for (int b = 0; b < kB; ++b) keys4(c.row, q, i0 + 4 * ((int64_t)b * T + tid), n, kk[b]);
    int nup = 0, ntie = 0;
#pragma unroll
    for (int b = 0; b < kB; ++b)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int64_t i = i0 + 4 * ((int64_t)b * T + tid) + t;
            const int dg = (int)(kk[b][t] >> kDigit0Shift);
            if (i < n) {
                nup += dg > bin;
                ntie += dg == bin;
            }
        }
    __syncthreads();
    const int lu = nup ? atomicAdd(&s_base[0], nup) : 0;
    const int lt = ntie ? atomicAdd(&s_base[1], ntie) : 0;
    __syncthreads();
    if (tid == 0) {
        s_base[2] = s_base[0] ? atomicAdd(&hist[kHistBins + 0], s_base[0]) : 0;
        s_base[3] = s_base[1] ? atomicAdd(&hist[kHistBins + 1], s_base[1]) : 0;
    }
    __syncthreads();
    int pu = s_base[2] + lu, pt = s_base[3] + lt;
    int32_t *out = c.idx + (int64_t)q * c.k;
    uint2 *cand = ws.cand + (int64_t)q * ws.cap;
#pragma unroll
    for (int b = 0; b < kB; ++b)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int64_t i = i0 + 4 * ((int64_t)b * T + tid) + t;
            if (i < n) {
                const int dg = (int)(kk[b][t] >> kDigit0Shift);
                if (dg > bin) {
                    out[pu++] = out_id(c.row, q, i);
                } else if (dg == bin) {
                    if (pt < ws.cap) cand[pt] = make_uint2(kk[b][t], (uint32_t)i);
                    ++pt;
                }
            }
        }
}

// The remaining digits among the tied rows, one workgroup per query.
__global__ __launch_bounds__(NT) void k_final(SelCall c, SelWorkspace ws)
{
    __shared__ Scratch<NT> sh;
    __shared__ uint32_t h0[kHistBins];
    __shared__ uint32_t ck[kCandCap];
    __shared__ int32_t ci[kCandCap];
    const int tid = threadIdx.x;
    const int q = blockIdx.x;
    const int n = query_n(c, q);
    const int K = min(n, c.k);
    int32_t *out = c.idx + (int64_t)q * c.k;
    if (K > 0) {
        const int32_t *hist = ws.hist + (int64_t)q * kHistStride;
        threshold_from_hist<NT>(hist, h0, K, sh);
        const int bin = sh.res[0];
        const int above = sh.res[1];
        if (bin >= 0) {
            const int nc = hist[kHistBins + 1];
            const uint2 *cand = ws.cand + (int64_t)q * ws.cap;
            if (tid == 0) sh.cnt[0] = above;
            const uint32_t prefix = (uint32_t)bin << kDigit0Shift;
            const uint32_t pmask = 0xFFFFFFFFu << kDigit0Shift;
            const uint32_t need = (uint32_t)(K - above);
            if (nc <= kCandCap && nc <= ws.cap) {
                for (int i0 = 0; i0 < nc; i0 += NT * 4) {
                    uint2 p[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = i0 + e * NT + tid;
                        p[e] = i < nc ? cand[i] : make_uint2(0u, 0u);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = i0 + e * NT + tid;
                        if (i < nc) {
                            ck[i] = p[e].x;
                            ci[i] = (int32_t)p[e].y;
                        }
                    }
                }
                __syncthreads();
                finish_levels<NT>(CandLds{ck, ci}, nc, prefix, pmask, need, out, c.row, q, sh);
            } else {
                finish_levels<NT>(RowGlobal{c.row, q}, n, prefix, pmask, need, out, c.row, q, sh);
            }
        }
    }
    for (int i = K + tid; i < c.k; i += NT) out[i] = -1;
    if (tid == 0) c.count[q] = K;
}

// Clears the per-query histograms and counters before a scoring kernel
// accumulates into them.
__global__ __launch_bounds__(256) void k_hist_clear(int32_t *hist, int64_t words)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (int64_t)gridDim.x * 256) hist[i] = 0;
}

bool use_filter(int64_t Q, int64_t max_n) { return max_n > kKeyCache && Q <= 64; }

int64_t cand_cap(int64_t Q, int64_t max_n) { return use_filter(Q, max_n) ? std::min<int64_t>(max_n, 65536) : 0; }

} // namespace

size_t sel_workspace_bytes(int64_t Q, int64_t max_n)
{
    size_t b = (size_t)Q * kHistStride * 4;
    b = (b + 255) & ~(size_t)255;
    return b + (size_t)Q * cand_cap(Q, max_n) * 8;
}

SelWorkspace sel_workspace_carve(void *base, int64_t Q, int64_t max_n)
{
    SelWorkspace w;
    w.hist = (int32_t *)base;
    size_t off = ((size_t)Q * kHistStride * 4 + 255) & ~(size_t)255;
    w.cand = (uint2 *)((uint8_t *)base + off);
    w.cap = cand_cap(Q, max_n);
    return w;
}

hipError_t launch_hist_clear(const SelWorkspace &ws, int64_t Q, hipStream_t s)
{
    const int64_t words = Q * kHistStride;
    const int64_t blocks = std::min<int64_t>((words + 255) / 256, 2048);
    hipLaunchKernelGGL(k_hist_clear, dim3((unsigned)blocks), dim3(256), 0, s, ws.hist, words);
    return hipGetLastError();
}

hipError_t launch_select(const SelCall &c, const SelWorkspace &ws, bool have_hist, hipStream_t s)
{
    if (c.Q <= 0) return hipSuccess;
    if (have_hist && use_filter(c.Q, c.max_n)) {
        const int64_t chunks = (c.max_n + kFilterChunk - 1) / kFilterChunk;
        hipLaunchKernelGGL(k_filter, dim3((unsigned)chunks, c.Q), dim3(kFilterThreads), 0, s, c, ws);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_final, dim3(c.Q), dim3(NT), 0, s, c, ws);
        return hipGetLastError();
    }
    if (have_hist)
        hipLaunchKernelGGL(k_select<true>, dim3(c.Q), dim3(NT), 0, s, c, ws);
    else
        hipLaunchKernelGGL(k_select<false>, dim3(c.Q), dim3(NT), 0, s, c, ws);
    return hipGetLastError();
}

} // namespace li

// Per-query top-k selection (gfx950).
//
// LatentIndex (paperlayer.ai summary of arXiv:2610.04635), §3.1/§4.1: every
// layer picks its own top-k rows (k = 2048), capped by the valid prefix
// (§C.4); the HS anchor picks its top-M candidates and its own top-k inside
// them (§3.2, §C.4).
//
// Scores become order-preserving uint32 keys and are selected by radix
// digits of 11, 11 and 10 bits (most significant first), on LDS histograms.
//   * Long rows (decode at 8K-128K): the first digit's histogram is built by
//     many workgroups per query (global atomics on 2048 bins); a filter pass
//     then writes every row whose first digit beats the threshold digit
//     straight to the output and compacts the rows that tie on it into a
//     candidate list; one workgroup per query resolves the last two digits
//     among the candidates in LDS.
//   * Short rows (HS followers, nested anchor selection, <= 16384): one
//     workgroup per query holds all keys in LDS and runs all three digits.
// Rows whose key equals the final threshold key are taken in arbitrary
// order, as many as the budget needs: equal scores are interchangeable.
#include "li_internal.hpp"

#include <algorithm>

namespace li {
namespace {

constexpr int kCtr = 4; // per-query counters: 0 out, 1 cand

__device__ __forceinline__ uint32_t key_at(const SelRow &r, int q, int64_t i)
{
    const int64_t j = r.gmap ? (int64_t)r.gmap[(int64_t)q * r.gld + i] : i;
    return score_key(r.S[(int64_t)q * r.ld + j]);
}

__device__ __forceinline__ int32_t out_id(const SelRow &r, int q, int64_t i)
{
    return r.omap ? r.omap[(int64_t)q * r.old + i] : (int32_t)i;
}

// Block-wide search on an LDS histogram: the bin b holding the `remaining`-th
// largest element, and `above` = elements in bins > b.  Writes res[0] = b
// (-1 if remaining exceeds the total), res[1] = above.  256 threads.
__device__ void find_bin(const uint32_t *h, int nbins, uint32_t remaining, uint32_t *scan, int *res)
{
    const int tid = threadIdx.x;
    const int per = nbins / kBlock;
    uint32_t sum = 0;
    for (int j = 0; j < per; ++j) sum += h[tid * per + j];
    if (tid == 0) res[0] = -1;
    scan[tid] = sum;
    __syncthreads();
    // inclusive suffix sums: scan[t] = sum over threads >= t
    for (int off = 1; off < kBlock; off <<= 1) {
        const uint32_t v = tid + off < kBlock ? scan[tid + off] : 0u;
        __syncthreads();
        scan[tid] += v;
        __syncthreads();
    }
    const uint32_t incl = scan[tid];
    const uint32_t excl = incl - sum;
    if (excl < remaining && incl >= remaining) {
        uint32_t acc = excl;
        for (int j = per - 1; j >= 0; --j) {
            const int bb = tid * per + j;
            if (acc + h[bb] >= remaining) {
                res[0] = bb;
                res[1] = (int)acc;
                break;
            }
            acc += h[bb];
        }
    }
    __syncthreads();
}

// Key/id sources for the in-block radix passes.
struct LdsKeys { // keys in LDS, id = index
    const uint32_t *k;
    __device__ uint32_t key(int64_t i) const { return k[i]; }
    __device__ int64_t id(int64_t i) const { return i; }
};
struct LdsPairs { // keys and ids in LDS
    const uint32_t *k;
    const int32_t *d;
    __device__ uint32_t key(int64_t i) const { return k[i]; }
    __device__ int64_t id(int64_t i) const { return d[i]; }
};
struct GlobalPairs { // candidate list in global memory
    const uint2 *p;
    __device__ uint32_t key(int64_t i) const { return p[i].x; }
    __device__ int64_t id(int64_t i) const { return (int32_t)p[i].y; }
};
struct RowKeys { // the query's whole score row
    SelRow r;
    int q;
    __device__ uint32_t key(int64_t i) const { return key_at(r, q, i); }
    __device__ int64_t id(int64_t i) const { return i; }
};

struct BlockScratch {
    uint32_t hist[kBins0];
    uint32_t scan[kBlock];
    int res[2];
    int cnt[2];
};

// Radix levels `level`..2 over m elements of `src` restricted to keys with
// (key & pmask) == prefix; emits the `remaining` best of them into
// out[out_base ...] (ids mapped through the row's omap).
template <class Src>
__device__ void radix_levels(const Src &src, int64_t m, int level, uint32_t prefix, uint32_t pmask,
                             uint32_t remaining, int32_t *out, int out_base, const SelRow &row, int q,
                             BlockScratch &sh)
{
    const int tid = threadIdx.x;
    if (tid == 0) sh.cnt[0] = out_base;
    __syncthreads();
    for (; level < 3 && remaining > 0; ++level) {
        const int shift = level == 0 ? 21 : (level == 1 ? 10 : 0);
        const int nb = level == 2 ? 1024 : 2048;
        const uint32_t dmask = (uint32_t)nb - 1u;
        for (int j = tid; j < nb; j += kBlock) sh.hist[j] = 0;
        __syncthreads();
        for (int64_t i = tid; i < m; i += kBlock) {
            const uint32_t key = src.key(i);
            if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & dmask], 1u);
        }
        __syncthreads();
        find_bin(sh.hist, nb, remaining, sh.scan, sh.res);
        const int bin = sh.res[0];
        const uint32_t above = (uint32_t)sh.res[1];
        if (bin < 0) break; // inconsistent counts: nothing sensible to emit
        for (int64_t i = tid; i < m; i += kBlock) {
            const uint32_t key = src.key(i);
            if ((key & pmask) == prefix && ((key >> shift) & dmask) > (uint32_t)bin) {
                const int o = atomicAdd(&sh.cnt[0], 1);
                out[o] = out_id(row, q, src.id(i));
            }
        }
        remaining -= above;
        prefix |= (uint32_t)bin << shift;
        pmask |= dmask << shift;
        __syncthreads();
    }
    if (remaining > 0 && level == 3) {
        if (tid == 0) sh.cnt[1] = 0;
        __syncthreads();
        for (int64_t i = tid; i < m; i += kBlock) {
            const uint32_t key = src.key(i);
            if (key == prefix) {
                const int slot = atomicAdd(&sh.cnt[1], 1);
                if ((uint32_t)slot < remaining) {
                    const int o = atomicAdd(&sh.cnt[0], 1);
                    out[o] = out_id(row, q, src.id(i));
                }
            }
        }
    }
    __syncthreads();
}

__device__ __forceinline__ void pad_and_count(int32_t *out, int K, int k, int32_t *count, int q)
{
    for (int i = K + threadIdx.x; i < k; i += kBlock) out[i] = -1;
    if (threadIdx.x == 0) count[q] = K;
}

// n, K per query; zero counters and histograms.
__global__ __launch_bounds__(256) void k_sel_prep(SelCall c, SelWorkspace ws)
{
    const int64_t tid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const int64_t words = (int64_t)c.Q * (kCtr + kBins0);
    for (int64_t i = tid; i < words; i += (int64_t)gridDim.x * kBlock) ws.ctr[i] = 0; // ctr then hist
    if (tid < c.Q) {
        const int q = (int)tid;
        int n;
        if (c.src_mode == kSrcCausal) {
            n = valid_rows(c.qpos[q], c.seq_lens[c.qseq[q]]);
        } else {
            n = c.cnt[q] < c.cnt_cap ? c.cnt[q] : c.cnt_cap;
            n = n > 0 ? n : 0;
        }
        if (n > c.max_n) n = (int)c.max_n; // the caller's bound sizes every buffer
        ws.nvalid[q] = n;
        ws.kq[q] = n < c.k ? n : c.k;
    }
}

// First-digit histogram, many workgroups per query.
__global__ __launch_bounds__(256) void k_sel_hist(SelCall c, SelWorkspace ws, int chunk)
{
    __shared__ uint32_t h[kBins0];
    const int q = blockIdx.y;
    const int n = ws.nvalid[q];
    const int64_t i0 = (int64_t)blockIdx.x * chunk;
    if (i0 >= n || ws.kq[q] == 0) return;
    for (int j = threadIdx.x; j < kBins0; j += kBlock) h[j] = 0;
    __syncthreads();
    const int64_t i1 = std::min<int64_t>(i0 + chunk, n);
    for (int64_t i = i0 + threadIdx.x; i < i1; i += kBlock) atomicAdd(&h[key_at(c.row, q, i) >> kDigit0Shift], 1u);
    __syncthreads();
    uint32_t *g = ws.hist + (int64_t)q * kBins0;
    for (int j = threadIdx.x; j < kBins0; j += kBlock)
        if (h[j]) atomicAdd(&g[j], h[j]);
}

// Rows above the threshold digit go to the output; rows on it to the
// candidate list.
template <int EPT>
__global__ __launch_bounds__(256) void k_sel_filter(SelCall c, SelWorkspace ws)
{
    __shared__ BlockScratch sh;
    __shared__ int s_base[4];
    const int q = blockIdx.y;
    const int n = ws.nvalid[q];
    const int K = ws.kq[q];
    const int64_t i0 = (int64_t)blockIdx.x * (EPT * kBlock);
    if (i0 >= n || K == 0) return;
    const uint32_t *g = ws.hist + (int64_t)q * kBins0;
    for (int j = threadIdx.x; j < kBins0; j += kBlock) sh.hist[j] = g[j];
    if (threadIdx.x < 4) s_base[threadIdx.x] = 0;
    __syncthreads();
    find_bin(sh.hist, kBins0, (uint32_t)K, sh.scan, sh.res);
    const int bin = sh.res[0];
    if (bin < 0) return;
    uint32_t keys[EPT];
    int nout = 0, ncand = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int64_t i = i0 + (int64_t)e * kBlock + threadIdx.x;
        keys[e] = i < n ? key_at(c.row, q, i) : 0u;
        const int dg = (int)(keys[e] >> kDigit0Shift);
        if (i < n) {
            nout += dg > bin;
            ncand += dg == bin;
        }
    }
    const int lo = nout ? atomicAdd(&s_base[0], nout) : 0;
    const int lc = ncand ? atomicAdd(&s_base[1], ncand) : 0;
    __syncthreads();
    if (threadIdx.x == 0) {
        s_base[2] = s_base[0] ? atomicAdd(&ws.ctr[q * kCtr + 0], s_base[0]) : 0;
        s_base[3] = s_base[1] ? atomicAdd(&ws.ctr[q * kCtr + 1], s_base[1]) : 0;
    }
    __syncthreads();
    int po = s_base[2] + lo, pc = s_base[3] + lc;
    int32_t *out = c.idx + (int64_t)q * c.k;
    uint2 *cand = ws.cand + (int64_t)q * ws.cap;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int64_t i = i0 + (int64_t)e * kBlock + threadIdx.x;
        if (i < n) {
            const int dg = (int)(keys[e] >> kDigit0Shift);
            if (dg > bin) {
                out[po++] = out_id(c.row, q, i);
            } else if (dg == bin) {
                if (pc < ws.cap) cand[pc] = make_uint2(keys[e], (uint32_t)i);
                ++pc;
            }
        }
    }
}

// Last two digits among the candidates, one workgroup per query.
__global__ __launch_bounds__(256) void k_sel_final(SelCall c, SelWorkspace ws)
{
    __shared__ BlockScratch sh;
    __shared__ uint32_t sk[kFinalLdsCap];
    __shared__ int32_t sd[kFinalLdsCap];
    const int q = blockIdx.x;
    const int K = ws.kq[q];
    int32_t *out = c.idx + (int64_t)q * c.k;
    if (K > 0) {
        const uint32_t *g = ws.hist + (int64_t)q * kBins0;
        for (int j = threadIdx.x; j < kBins0; j += kBlock) sh.hist[j] = g[j];
        __syncthreads();
        find_bin(sh.hist, kBins0, (uint32_t)K, sh.scan, sh.res);
        const int bin = sh.res[0];
        const int above = sh.res[1];
        __syncthreads();
        if (bin >= 0) {
            const uint32_t prefix = (uint32_t)bin << kDigit0Shift;
            const uint32_t pmask = 0xFFE00000u;
            const uint32_t need = (uint32_t)(K - above);
            const int64_t nc = ws.ctr[q * kCtr + 1];
            const uint2 *cand = ws.cand + (int64_t)q * ws.cap;
            // The list holds min(nc, cap) entries: use it only when complete.
            if (nc <= ws.cap && nc <= kFinalLdsCap) {
                for (int64_t i = threadIdx.x; i < nc; i += kBlock) {
                    const uint2 p = cand[i];
                    sk[i] = p.x;
                    sd[i] = (int32_t)p.y;
                }
                __syncthreads();
                radix_levels(LdsPairs{sk, sd}, nc, 1, prefix, pmask, need, out, above, c.row, q, sh);
            } else if (nc <= ws.cap) {
                radix_levels(GlobalPairs{cand}, nc, 1, prefix, pmask, need, out, above, c.row, q, sh);
            } else {
                radix_levels(RowKeys{c.row, q}, ws.nvalid[q], 1, prefix, pmask, need, out, above, c.row, q, sh);
            }
        }
    }
    pad_and_count(out, K, c.k, c.count, q);
}

// Whole selection in one workgroup per query (n <= kSmallCap).
__global__ __launch_bounds__(256) void k_sel_small(SelCall c, SelWorkspace ws)
{
    __shared__ BlockScratch sh;
    __shared__ uint32_t sk[kSmallCap];
    const int q = blockIdx.x;
    const int n = ws.nvalid[q];
    const int K = ws.kq[q];
    int32_t *out = c.idx + (int64_t)q * c.k;
    if (K > 0) {
        for (int64_t i = threadIdx.x; i < n; i += kBlock) sk[i] = key_at(c.row, q, i);
        __syncthreads();
        radix_levels(LdsKeys{sk}, n, 0, 0u, 0u, (uint32_t)K, out, 0, c.row, q, sh);
    }
    pad_and_count(out, K, c.k, c.count, q);
}

} // namespace

size_t sel_workspace_bytes(int64_t Q, int64_t max_n)
{
    const int64_t cap = std::max<int64_t>(1, std::min<int64_t>(max_n, Q <= 64 ? 65536 : 8192));
    size_t b = 0;
    b += (size_t)Q * 4 * 2;                         // nvalid, kq
    b = (b + 255) & ~(size_t)255;
    b += (size_t)Q * (kCtr + kBins0) * 4;           // ctr + hist
    b = (b + 255) & ~(size_t)255;
    b += (size_t)Q * cap * 8;                       // candidates
    return b;
}

SelWorkspace sel_workspace_carve(void *base, int64_t Q, int64_t max_n)
{
    const int64_t cap = std::max<int64_t>(1, std::min<int64_t>(max_n, Q <= 64 ? 65536 : 8192));
    uint8_t *p = (uint8_t *)base;
    SelWorkspace w;
    w.nvalid = (int32_t *)p;
    w.kq = w.nvalid + Q;
    size_t off = ((size_t)Q * 8 + 255) & ~(size_t)255;
    w.ctr = (int32_t *)(p + off);
    w.hist = (uint32_t *)(w.ctr + Q * kCtr);
    off += (size_t)Q * (kCtr + kBins0) * 4;
    off = (off + 255) & ~(size_t)255;
    w.cand = (uint2 *)(p + off);
    w.cap = cap;
    return w;
}

hipError_t launch_sel_prep(const SelCall &c, const SelWorkspace &ws, hipStream_t s)
{
    const int64_t words = (int64_t)c.Q * (kCtr + kBins0);
    int64_t blocks = std::max<int64_t>((words + kBlock - 1) / kBlock, (c.Q + kBlock - 1) / kBlock);
    blocks = std::min<int64_t>(blocks, 4096);
    hipLaunchKernelGGL(k_sel_prep, dim3((unsigned)blocks), dim3(kBlock), 0, s, c, ws);
    return hipGetLastError();
}

hipError_t launch_select(const SelCall &c, const SelWorkspace &ws, hipStream_t s)
{
    if (c.Q <= 0) return hipSuccess;
    if (c.max_n <= kSmallCap) {
        hipLaunchKernelGGL(k_sel_small, dim3(c.Q), dim3(kBlock), 0, s, c, ws);
        return hipGetLastError();
    }
    constexpr int EPT = 16;
    const int chunk = EPT * kBlock;
    const int64_t chunks = (c.max_n + chunk - 1) / chunk;
    hipLaunchKernelGGL(k_sel_hist, dim3((unsigned)chunks, c.Q), dim3(kBlock), 0, s, c, ws, chunk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_sel_filter<EPT>, dim3((unsigned)chunks, c.Q), dim3(kBlock), 0, s, c, ws);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_sel_final, dim3(c.Q), dim3(kBlock), 0, s, c, ws);
    return hipGetLastError();
}

} // namespace li

// Latent-row scoring kernels (gfx950).
//
// LatentIndex (paperlayer.ai summary of arXiv:2610.04635), §3.1 and §B.2:
// every layer scores the shared latent cache directly with its absorbed
// query, I(j) = sum_h w_h * max(0, qt_h . c_j).  With 64 heads x r = 256
// against N rows this is a dense (heads x r) . (r x rows) contraction, so
// it runs on MFMA: v_mfma_f32_32x32x16_bf16 with
//   A (32 heads x 16 k)  = absorbed query, held in VGPRs for the whole kernel,
//   B (16 k x 32 rows)   = a 32-row latent tile staged in LDS,
//   D (32 heads x 32 rows) fp32; lane l owns row l%32 and 16 heads of it,
// so the ReLU, the head weights and the head sum are a per-lane loop plus one
// exchange between the two lane halves.
//
// Latent tiles travel HBM -> LDS with global_load_lds_dwordx4 (no VGPR
// staging).  Each 1 KiB DMA instruction copies 512/r whole rows; within a
// row the 16-byte chunks are XOR-swizzled by the row index so that the MFMA
// operand reads (32 rows, same chunk) hit distinct LDS banks.
#include "li_internal.hpp"

#include <algorithm>

namespace li {
namespace {

constexpr int kGatherTiles = 16; // max tiles per wave in gather mode (row offsets kept in LDS)

// LDS-typed pointers keep every access a ds_* instruction (a generic pointer
// would become a flat access that also waits on global memory).
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef const __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef const __attribute__((address_space(4))) int32_t const_i32_t;

__device__ __forceinline__ void dma16(const void *g, lds_u8 *lds_uniform)
{
    __builtin_amdgcn_global_load_lds(g, (lds_void_t *)lds_uniform, 16, 0, 0);
}

// Workgroup barrier without the global-memory fences of __syncthreads():
// outstanding DMA loads stay in flight across it.  This wave's LDS reads are
// complete before it arrives.
__device__ __forceinline__ void wg_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void wait_lds()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

__device__ __forceinline__ int64_t min64(int64_t x, int64_t y) { return x < y ? x : y; }

__device__ __forceinline__ int64_t shfl64(int64_t v, int src)
{
    int lo = __shfl((int)(uint32_t)(uint64_t)v, src);
    int hi = __shfl((int)(uint32_t)((uint64_t)v >> 32), src);
    return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo);
}

// Dynamic-count wait (the count must be an immediate).
template <int NIW>
__device__ __forceinline__ void wait_after(int tiles_after)
{
    switch (tiles_after) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<NIW>(); break;
    case 2: wait_vmcnt<2 * NIW < 63 ? 2 * NIW : 0>(); break;
    default: wait_vmcnt<3 * NIW < 63 ? 3 * NIW : 0>(); break;
    }
}

// LDS byte offset of 16-byte chunk c of tile row nr.
template <int R>
__device__ __forceinline__ int lds_chunk(int nr, int c)
{
    constexpr int CH = R / 8;
    return (nr * CH + (c ^ (nr % CH))) * 16;
}

// Absorbed-query fragments (MFMA A operand) and per-lane head weights.
template <int R, int HB>
struct QueryRegs {
    bf16x8 a[HB][R / 16];
    float w[HB][16];

    __device__ __forceinline__ void load(const u16 *qt, const float *wq, int H)
    {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            const int h = hb * 32 + (lane & 31);
#pragma unroll
            for (int s = 0; s < R / 16; ++s) {
                if (h < H) {
                    a[hb][s] = *(const bf16x8 *)(qt + (int64_t)h * R + s * 16 + (lane >> 5) * 8);
                } else {
                    bf16x8 z = {};
                    a[hb][s] = z;
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int hh = hb * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                w[hb][r] = hh < H ? wq[hh] : 0.0f;
            }
        }
    }
};

// Score of tile row (lane % 32), complete in every lane.
template <int R, int HB>
__device__ __forceinline__ float tile_score(const lds_u8 *buf, const QueryRegs<R, HB> &qr)
{
    const int lane = threadIdx.x & 63;
    const int nr = lane & 31, g = lane >> 5;
    f32x16 acc[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        f32x16 z = {};
        acc[hb] = z;
    }
#pragma unroll
    for (int s = 0; s < R / 16; ++s) {
        const bf16x8 b = *(lds_bf16x8 *)(buf + lds_chunk<R>(nr, 2 * s + g));
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
            acc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qr.a[hb][s], b, acc[hb], 0, 0, 0);
    }
    float p = 0.0f;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            p += qr.w[hb][r] * fmaxf(acc[hb][r], 0.0f);
    p += __shfl_xor(p, 32);
    return p;
}

// One wave copies a 32-row tile whose rows start at the given pool element
// offsets (rowoff of tile row i lives in lane i).
template <int R>
__device__ __forceinline__ void issue_tile_rows(const u16 *pool, int64_t rowoff, lds_u8 *buf)
{
    constexpr int CH = R / 8, NI = R / 16;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int ii = 0; ii < NI; ++ii) {
        const int p = ii * 64 + lane;
        const int nr = p / CH, cs = p % CH;
        const int c = cs ^ (nr % CH);
        const int64_t off = shfl64(rowoff, nr);
        dma16(pool + off + c * 8, buf + ii * 1024);
    }
}

// Part `part` of `parts` of a 32-row tile of physically contiguous rows.
template <int R>
__device__ __forceinline__ void issue_tile_contig(const u16 *tile_base, lds_u8 *buf, int part, int parts)
{
    constexpr int CH = R / 8, NI = R / 16;
    const int lane = threadIdx.x & 63;
    const int per = NI / parts;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        if (j < per) {
            const int ii = part * per + j;
            const int p = ii * 64 + lane;
            const int nr = p / CH, cs = p % CH;
            const int c = cs ^ (nr % CH);
            dma16(tile_base + nr * R + c * 8, buf + ii * 1024);
        }
    }
}

// ---------------------------------------------------------------------------
// Decode: few queries, long rows.  Workgroup = 4 waves of one query; each
// wave streams its own tiles (rows row0 + (wave + 4 i) * 32) through two LDS
// buffers, keeping one tile in flight while it computes the other.
// ---------------------------------------------------------------------------
template <int R, int HB, bool GATHER>
__global__ __launch_bounds__(256) void k_score_decode(ScoreArgs a, int tiles_per_wave)
{
    constexpr int TILE_BYTES = kTile * R * 2;
    constexpr int NI = R / 16;
    __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[4 * 2 * TILE_BYTES];
    __shared__ int64_t s_off[GATHER ? 4 * kGatherTiles * kTile : 1];
    lds_u8 *lds = (lds_u8 *)lds_raw;

    const int q = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int b = a.qseq[q];
    int n = GATHER ? min(a.cand_count[q], (int)a.cand_ld) : valid_rows(a.qpos[q], a.seq_lens[b]);
    n = (int)min64(n, a.max_rows);
    const int64_t rows_per_wg = (int64_t)4 * tiles_per_wave * kTile;
    const int64_t row0 = (int64_t)blockIdx.x * rows_per_wg;
    if (row0 >= n) return;
    // tiles of this wave: t = row0 + (wv + 4 i) * 32, i < nt
    const int64_t first = row0 + (int64_t)wv * kTile;
    int nt = 0;
    if (first < n) nt = (int)min64(tiles_per_wave, (n - first + 4 * kTile - 1) / (4 * kTile));

    const u16 *pool = (const u16 *)a.pool;
    const_i32_t *bt = (const_i32_t *)(a.bt + (int64_t)b * a.max_pages);
    lds_u8 *const wbuf = lds + wv * 2 * TILE_BYTES;
    auto buf = [&](int i) -> lds_u8 * { return wbuf + (i & 1) * TILE_BYTES; };

    auto tile_row0 = [&](int i) -> int64_t { return first + (int64_t)i * 4 * kTile; };
    // element offset in the pool of row (lane & 31) of tile i
    auto gather_off = [&](int i) -> int64_t {
        int64_t j = tile_row0(i) + (lane & 31);
        j = j < n ? j : n - 1;
        const int pos = a.cand[(int64_t)q * a.cand_ld + j];
        const int page = a.bt[(int64_t)b * a.max_pages + (pos >> 6)];
        return ((int64_t)page * kPage + (pos & 63)) * R;
    };
    auto issue = [&](int i) {
        if constexpr (GATHER) {
            issue_tile_rows<R>(pool, s_off[(wv * kGatherTiles + i) * kTile + (lane & 31)], buf(i));
        } else {
            const int64_t t0 = tile_row0(i);
            const int page = bt[t0 >> 6];
            issue_tile_contig<R>(pool + ((int64_t)page * kPage + (t0 & 63)) * R, buf(i), 0, 1);
        }
    };

    if constexpr (GATHER) {
        // Row offsets of every tile of this wave, resolved once up front.
        for (int i = 0; i < nt; ++i) {
            const int64_t off = gather_off(i);
            if (lane < 32) s_off[(wv * kGatherTiles + i) * kTile + lane] = off;
        }
        wait_vmcnt<0>();
        wait_lds();
    }

    if (nt > 0) issue(0);
    QueryRegs<R, HB> qr;
    qr.load((const u16 *)a.qt + (int64_t)q * a.H * R, a.w + (int64_t)q * a.H, a.H);
    if (nt > 1) issue(1);

    float *out = a.out + (int64_t)q * a.out_ld;
    for (int i = 0; i < nt; ++i) {
        if (i + 1 < nt) wait_vmcnt<NI>();
        else wait_vmcnt<0>();
        const float p = tile_score<R, HB>(buf(i), qr);
        const int64_t j = tile_row0(i) + lane;
        if (lane < 32 && j < n) out[j] = p;
        if (i + 2 < nt) {
            wait_lds(); // this wave's reads of the buffer are done before it is refilled
            issue(i + 2);
        }
    }
}

// ---------------------------------------------------------------------------
// Prefill: many queries per sequence.  Workgroup = 4 consecutive queries,
// one per wave; the 4 waves share every latent tile (one DMA per tile,
// split across the waves) through an NBUF-deep LDS ring.  Queries of a
// workgroup that sit in different sequences are served in separate passes.
// ---------------------------------------------------------------------------
template <int R, int HB, int NBUF>
__global__ __launch_bounds__(256) void k_score_prefill(ScoreArgs a, int tiles_per_split)
{
    constexpr int TILE_BYTES = kTile * R * 2;
    constexpr int NI = R / 16;
    constexpr int NIW = NI / 4;
    static_assert(NIW >= 1, "tile must split over 4 waves");
    __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[NBUF * TILE_BYTES];
    lds_u8 *lds = (lds_u8 *)lds_raw;

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int qbase = blockIdx.x * 4;
    const_i32_t *qseq = (const_i32_t *)a.qseq;
    const_i32_t *qpos = (const_i32_t *)a.qpos;
    const_i32_t *slen = (const_i32_t *)a.seq_lens;
    int sb[4], sn[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int qq = qbase + u;
        sb[u] = qq < a.Q ? qseq[qq] : -1;
        sn[u] = qq < a.Q ? (int)min64(valid_rows(qpos[qq], slen[sb[u]]), a.max_rows) : 0;
    }
    const int q = qbase + wv;
    int my_b = -1, my_n = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u)
        if (u == wv) {
            my_b = sb[u];
            my_n = sn[u];
        }
    QueryRegs<R, HB> qr;
    if (q < a.Q) {
        qr.load((const u16 *)a.qt + (int64_t)q * a.H * R, a.w + (int64_t)q * a.H, a.H);
    } else {
        qr.load((const u16 *)a.qt, a.w, 0); // zero fragments
    }
    float *out = a.out + (int64_t)(q < a.Q ? q : 0) * a.out_ld;
    const u16 *pool = (const u16 *)a.pool;

#pragma unroll 1
    for (int u = 0; u < 4; ++u) {
        const int b = sb[u];
        bool skip = b < 0;
        int nmax = 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            if (v < u && sb[v] == b) skip = true;
            if (sb[v] == b) nmax = max(nmax, sn[v]);
        }
        if (skip) continue;
        const bool active = (my_b == b) && (q < a.Q);
        const int ntiles_all = (nmax + kTile - 1) / kTile;
        const int ts = blockIdx.y * tiles_per_split;
        const int te = min(ts + tiles_per_split, ntiles_all);
        if (ts >= te) continue;
        const int nt = te - ts;
        const_i32_t *bt = (const_i32_t *)(a.bt + (int64_t)b * a.max_pages);
        auto issue = [&](int i) {
            const int64_t t0 = (int64_t)(ts + i) * kTile;
            const int page = bt[t0 >> 6];
            issue_tile_contig<R>(pool + ((int64_t)page * kPage + (t0 & 63)) * R,
                                 lds + (i % NBUF) * TILE_BYTES, wv, 4);
        };
        for (int i = 0; i < NBUF - 1 && i < nt; ++i) issue(i);
#pragma unroll 1
        for (int i = 0; i < nt; ++i) {
            if (i + NBUF - 1 < nt) issue(i + NBUF - 1);
            wait_after<NIW>(min(NBUF - 1, nt - 1 - i));
            wg_barrier();
            if (active) {
                const float p = tile_score<R, HB>(lds + (i % NBUF) * TILE_BYTES, qr);
                const int j = (ts + i) * kTile + lane;
                if (lane < 32 && j < my_n) out[j] = p;
            }
            wg_barrier();
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 latent (any r <= 256): plain VALU dot products, one row per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_score_f32(ScoreArgs a, int R)
{
    __shared__ float sq[64 * 256];
    __shared__ float sw[64];
    const int q = blockIdx.y;
    const int b = a.qseq[q];
    int n = a.cand ? min(a.cand_count[q], (int)a.cand_ld) : valid_rows(a.qpos[q], a.seq_lens[b]);
    n = (int)min64(n, a.max_rows);
    const int64_t row0 = (int64_t)blockIdx.x * 256;
    if (row0 >= n) return;
    const float *qt = (const float *)a.qt + (int64_t)q * a.H * R;
    for (int i = threadIdx.x; i < a.H * R; i += 256) sq[i] = qt[i];
    for (int i = threadIdx.x; i < a.H; i += 256) sw[i] = a.w[(int64_t)q * a.H + i];
    __syncthreads();
    const int64_t j = row0 + threadIdx.x;
    if (j >= n) return;
    const int pos = a.cand ? a.cand[(int64_t)q * a.cand_ld + j] : (int)j;
    const int page = a.bt[(int64_t)b * a.max_pages + (pos >> 6)];
    const float *row = (const float *)a.pool + ((int64_t)page * kPage + (pos & 63)) * R;
    float s = 0.0f;
    for (int h = 0; h < a.H; ++h) {
        float dot = 0.0f;
        for (int t = 0; t < R; ++t) dot = fmaf(sq[h * R + t], row[t], dot);
        s = fmaf(sw[h], fmaxf(dot, 0.0f), s);
    }
    a.out[(int64_t)q * a.out_ld + j] = s;
}

template <int R, int HB>
hipError_t launch_bf16(const ScoreArgs &a, bool prefill, int64_t max_rows, hipStream_t s)
{
    const int64_t tiles = (max_rows + kTile - 1) / kTile;
    if (prefill) {
        constexpr int NBUF = R == 256 ? 4 : 6;
        const int qblocks = (a.Q + 3) / 4;
        int splits = 1;
        if (qblocks < 512) splits = (int)std::min<int64_t>((512 + qblocks - 1) / qblocks, tiles);
        if (splits < 1) splits = 1;
        const int tps = (int)((tiles + splits - 1) / splits);
        splits = (int)((tiles + tps - 1) / tps);
        hipLaunchKernelGGL((k_score_prefill<R, HB, NBUF>), dim3(qblocks, splits), dim3(256), 0, s, a, tps);
        return hipGetLastError();
    }
    // decode: aim for ~2 rounds of one workgroup per CU
    const int64_t want_wgs = 512;
    int64_t per_q = (want_wgs + a.Q - 1) / a.Q;
    int64_t tpw = (tiles + 4 * per_q - 1) / (4 * per_q);
    if (tpw < 1) tpw = 1;
    if (tpw > 64) tpw = 64;
    if (a.cand && tpw > kGatherTiles) tpw = kGatherTiles;
    const int64_t wgs = (tiles + 4 * tpw - 1) / (4 * tpw);
    if (a.cand)
        hipLaunchKernelGGL((k_score_decode<R, HB, true>), dim3((unsigned)wgs, a.Q), dim3(256), 0, s, a, (int)tpw);
    else
        hipLaunchKernelGGL((k_score_decode<R, HB, false>), dim3((unsigned)wgs, a.Q), dim3(256), 0, s, a, (int)tpw);
    return hipGetLastError();
}

template <int R>
hipError_t launch_r(const ScoreArgs &a, bool prefill, int64_t max_rows, hipStream_t s)
{
    if (a.H <= 32) return launch_bf16<R, 1>(a, prefill, max_rows, s);
    return launch_bf16<R, 2>(a, prefill, max_rows, s);
}

} // namespace

hipError_t launch_score(const ScoreArgs &a, int r, bool bf16, bool many_queries_per_seq, int64_t max_rows,
                        hipStream_t s)
{
    if (a.Q <= 0 || max_rows <= 0) return hipSuccess;
    const bool prefill = many_queries_per_seq && a.cand == nullptr;
    if (!bf16) {
        const int64_t wgs = (max_rows + 255) / 256;
        hipLaunchKernelGGL(k_score_f32, dim3((unsigned)wgs, a.Q), dim3(256), 0, s, a, r);
        return hipGetLastError();
    }
    switch (r) {
    case 64: return launch_r<64>(a, prefill, max_rows, s);
    case 128: return launch_r<128>(a, prefill, max_rows, s);
    case 256: return launch_r<256>(a, prefill, max_rows, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace li

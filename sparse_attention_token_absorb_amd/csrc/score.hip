// Latent-row scoring kernels (gfx950).
//
// LatentIndex (paperlayer.ai summary of arXiv:2610.04635), §3.1 and §B.2:
// every layer scores the shared latent cache directly with its absorbed
// query, I(j) = sum_h w_h * max(0, qt_h . c_j).  With 64 heads x r = 256
// against N rows this is a dense (heads x r) . (r x rows) contraction, so
// it runs on MFMA: v_mfma_f32_32x32x16_bf16 with
//   A (32 heads x 16 k)  = absorbed query, held in VGPRs for the whole kernel,
//   B (16 k x 32 rows)   = latent rows staged in LDS,
//   D (32 heads x 32 rows) fp32; lane l owns row l%32 and 16 heads of it,
// so the ReLU, the head weights and the head sum are a per-lane loop plus one
// exchange between the two lane halves.
//
// Latent rows travel HBM -> LDS with global_load_lds_dwordx4 (no VGPR
// staging); within a row the 16-byte pieces are XOR-swizzled by the row
// index so that the MFMA operand reads (32 rows, same piece) hit distinct
// LDS banks.  The epilogue also counts each score's first radix digit
// (key >> 20) into an LDS histogram that is merged into the query's global
// histogram at the end (only non-empty bins), so the top-k selection that
// follows starts from a known threshold bin.
#include "li_device.hpp"
#include "li_internal.hpp"
#include "li_probe.hpp"
#include "li_tail.hpp"
#include "li_timing.hpp"

#include <stdlib.h>
#include <string.h>

#include <algorithm>

namespace li {

#ifdef LI_PHASE_PROBE
__device__ uint64_t g_phase_bf16[kProbeWaves * kProbeWords]; // phase records (instrumented build only)
#endif
namespace {

constexpr int kGatherTiles = 16; // max tiles per wave in gather mode (row offsets kept in LDS)
constexpr int kMaxTilesPerWave = 64; // max tiles per wave of the contiguous LDS-ring decode kernel
constexpr int kGatherBtLds = 4096;    // block-table row entries kept in LDS in gather mode (262144 rows)
constexpr int kVrMaxTiles = 32;  // max tiles per wave of the register-staged decode kernel
constexpr int kPrefillMaxTiles = 2048; // max tiles per prefill split (their page ids sit in LDS)

template <int R, int HB>
struct QueryRegs {
    bf16x8 a[HB][R / 16];
    float w[HB][16];
    f32x16 b[HB]; // accumulator start values: each head's absorbed decoder bias (0 without one)

    // Staged through LDS (see stage_query): row h of the query lives in the
    // last ring slot of wave h / 16, row-local piece c at c ^ (h % PR); the
    // head weights in s_w.  Heads past H read as zero.
    template <int NB, int CHUNK>
    __device__ __forceinline__ void from_lds(const lds_u8 *ring, const lds_f32 *s_w, const lds_f32 *s_b, bool has_bias,
                                             int H)
    {
        constexpr int PR = R / 8; // 16-byte pieces per query row
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            const int h = hb * 32 + (lane & 31);
            const lds_u8 *row = ring + ((h >> 4) * NB + NB - 1) * CHUNK + (h & 15) * PR * 16;
#pragma unroll
            for (int s = 0; s < R / 16; ++s) {
                const int c = 2 * s + (lane >> 5);
                bf16x8 v = *(const lds_bf16x8 *)(row + (c ^ (h & (PR - 1))) * 16);
                if (h >= H) {
                    bf16x8 z = {};
                    v = z;
                }
                a[hb][s] = v;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int hh = hb * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                w[hb][r] = hh < H ? s_w[hh] : 0.0f;
                b[hb][r] = has_bias && hh < H ? s_b[hh] : 0.0f;
            }
        }
    }

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

// All R/16 MFMA steps over one full-width tile in LDS, with the B fragments
// read D steps ahead of their use so LDS latency hides behind the MFMAs.
// ZC: the accumulators start from zero (the first step takes a constant 0
// as its addend; acc is not read).
template <int R, int HB, int CH, int D, bool ZC = false>
__device__ __forceinline__ void mfma_tile_prefetch(const lds_u8 *buf, const QueryRegs<R, HB> &qr,
                                                   f32x16 (&acc)[HB])
{
    constexpr int KS = R / 16;
    constexpr int DD = D < KS ? D : KS;
    const int lane = threadIdx.x & 63;
    const int nr = lane & 31, g = lane >> 5;
    auto frag = [&](int s) -> bf16x8 {
        const int c = 2 * s + g;
        return *(lds_bf16x8 *)(buf + (nr * CH + (c ^ (nr % CH))) * 16);
    };
    bf16x8 b[DD];
#pragma unroll
    for (int s = 0; s < DD; ++s) b[s] = frag(s);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const bf16x8 cur = b[s % DD];
        if (s + DD < KS) b[s % DD] = frag(s + DD);
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            const f32x16 zero = {};
            acc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qr.a[hb][s], cur, ZC && s == 0 ? zero : acc[hb], 0, 0,
                                                              0);
        }
    }
    // Keep that order in the schedule: the first DD reads, then per step
    // its HB MFMAs followed by the read for step s + DD.
    __builtin_amdgcn_sched_group_barrier(0x100, DD, 0);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, HB, 0);
        if (s + DD < KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
}

// Copy `NIC` KiB of a 32-row tile (CH pieces of 16 B per row, starting at
// column `col0`) into LDS: instruction ii moves 64/CH rows.  rowoff(nr)
// gives the pool element offset of tile row nr.
template <int R, int CH, int NIC, bool NT = false, class RowOff>
__device__ __forceinline__ void issue_rows(const u16 *pool, const RowOff &rowoff, int col0, lds_u8 *buf, int ii0,
                                           int nii)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < NIC; ++j) {
        if (j < nii) {
            const int ii = ii0 + j;
            const int p = ii * 64 + lane;
            const int nr = p / CH, cs = p % CH;
            const int c = cs ^ (nr % CH);
            dma16p<NT>(pool + rowoff(nr) + col0 + c * 8, buf + ii * 1024);
        }
    }
}

// The query's rows into LDS, once per workgroup: wave w moves rows
// 16w .. 16w+15 (HB * 32 rows in all; rows past H repeat row H-1 and are
// zeroed when read) into the last slot of its ring, which the stream does not
// touch before its (NB-1)-th chunk; wave 0 also moves the head weights and
// wave 1 the heads' decoder biases (when there are any).
// Returns the number of loads this wave issued.
template <int R, int HB, int NB, int CHUNK>
__device__ __forceinline__ int stage_query(const u16 *qt, const float *wq, const float *bq, int H, lds_u8 *ring,
                                           lds_f32 *s_w, lds_f32 *s_b)
{
    constexpr int PR = R / 8;
    constexpr int NIC = R / 32; // 16 query rows of 2R bytes, 1 KiB per instruction
    static_assert(CHUNK >= 32 * R, "a ring slot holds 16 query rows");
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int issued = 0;
    if (wv * 16 < HB * 32) {
        lds_u8 *slot = ring + (wv * NB + NB - 1) * CHUNK;
#pragma unroll
        for (int ii = 0; ii < NIC; ++ii) {
            const int p = ii * 64 + lane;
            const int hl = p / PR, cs = p % PR;
            const int h = wv * 16 + hl;
            const int hs = h < H ? h : H - 1;
            dma16(qt + (int64_t)hs * R + (cs ^ (h & (PR - 1))) * 8, slot + ii * 1024);
        }
        issued = NIC;
    }
    if (wv == 0) {
        dma4(wq + (lane < H ? lane : H - 1), (lds_u8 *)s_w);
        ++issued;
    }
    if (wv == 1 && bq) {
        dma4(bq + (lane < H ? lane : H - 1), (lds_u8 *)s_b);
        ++issued;
    }
    return issued;
}

// ---------------------------------------------------------------------------
// Decode: few queries, long rows.  Workgroup = 4 waves of one query; wave w
// streams tiles row0 + (w + 4 i) * 32, so the workgroup covers a contiguous
// range of rows.  Each tile moves as CPT chunks of 32 rows x r/CPT columns
// (two half-width chunks at r = 256, where a whole tile is 16 KiB; whole
// tiles at r <= 128) through a per-wave ring of NB chunk buffers, so NB-1
// chunks stay in flight while the wave computes.
//
// Scores stay in LDS until the stream is done and leave in one coalesced
// burst per workgroup: score stores spread through the stream interleave
// writes with the HBM read stream, which measured 7% slower on a 1 GiB pool.
// NT: the latent rows are read with the non-temporal policy, for launches
// that stream more than the last-level cache can keep (a pool read once
// per launch gains nothing from allocating in it, and evicts everything else).
// With one wave per SIMD, a chunk's vector work delays the next DMA issue:
// over contiguous prefixes the DMA takes a scalar base plus fixed lane
// offsets, and the chunk loop is unrolled over the ring (and the chunks of
// a tile) so that every LDS address is a fixed lane offset plus an immediate.
// ---------------------------------------------------------------------------
template <int R, int HB, bool GATHER, int NB, int CPT, bool NT, bool BIAS>
__global__ __launch_bounds__(256) void k_score_decode(ScoreArgs a, int tiles_per_wave)
{
    static_assert(CPT == 1 || CPT == 2, "chunks per tile");
    constexpr int WC = R / CPT;                 // columns per chunk
    constexpr int CHUNK = kTile * WC * 2;       // bytes per chunk
    constexpr int NIC = CHUNK / 1024;           // DMA instructions per chunk
    constexpr int CH = WC / 8;                  // 16-byte pieces per chunk row
    constexpr int KSH = WC / 16;                // MFMA k-steps per chunk
    constexpr int MAXT = GATHER ? kGatherTiles : kMaxTilesPerWave; // tiles per wave (scores kept in LDS)
    __shared__ __attribute__((aligned(1024))) uint8_t ring_raw[4 * NB * CHUNK];
    __shared__ int32_t s_row[GATHER ? 4 * kGatherTiles * kTile : 1];
    __shared__ uint32_t s_hist[kHistBins];
    __shared__ float s_out[4 * MAXT * kTile];
    __shared__ int32_t s_pg[GATHER ? 1 : 4 * 64];
    __shared__ int32_t s_bt[GATHER ? kGatherBtLds : 1];
    __shared__ float s_w[64];
    __shared__ float s_b[64];

    const int q = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    LI_PHASE_DECL;
    LI_PHASE_START;
    const int64_t row0 = (int64_t)blockIdx.x * 4 * tiles_per_wave * kTile;
    const int64_t first = row0 + (int64_t)wv * kTile;
    auto tile_row0 = [&](int i) -> int64_t { return first + (int64_t)i * 4 * kTile; };
    // This wave's tile count if the query had max_rows rows (its real count,
    // known once the row count arrives, is at most that).
    const int nt_max =
        first < a.max_rows ? (int)min64(tiles_per_wave, (a.max_rows - first + 4 * kTile - 1) / (4 * kTile)) : 0;

    // Start-up is a chain of dependent loads (sequence id, then page ids and
    // the row count).  In contiguous mode lane i of a wave holds the page id
    // of the wave's tile i (the launcher keeps tiles_per_wave <= 64), so the
    // stream reads page ids from a register.  A decode batch usually has
    // query q in sequence q: that block-table row is requested first, by LDS
    // DMA, before the sequence id is known and ahead of the query staging,
    // and used if the guess was right.  The query's rows, weights and biases
    // go next (into LDS, read back once all have landed).  The first chunks
    // are issued as soon as the page ids are in, before the query and the
    // row count: a page id that is not in use is clamped into the pool, and
    // what such a chunk brings in is never scored.
    const int b_guess = q < a.batch ? q : 0;
    if constexpr (!GATHER) {
        const int pidx = (int)min64(tile_row0(lane < nt_max ? lane : 0) >> 6, a.max_pages - 1);
        dma4(a.bt + (int64_t)b_guess * a.max_pages + pidx, (lds_u8 *)(s_pg + wv * 64));
    } else if (a.max_pages <= kGatherBtLds) {
        // gather mode: the guessed sequence's whole block-table row, so that
        // the candidates' page lookups read LDS instead of waiting on memory
        for (int i = wv; i * 64 < a.max_pages; i += 4) {
            const int pidx = min(i * 64 + lane, a.max_pages - 1);
            dma4(a.bt + (int64_t)b_guess * a.max_pages + pidx, (lds_u8 *)(s_bt + i * 64));
        }
    }
    lds_u8 *const ring_all = (lds_u8 *)ring_raw;
    const int staged = stage_query<R, HB, NB, CHUNK>((const u16 *)a.qt + (int64_t)q * a.H * R, a.w + (int64_t)q * a.H,
                                                     a.bias ? a.bias + (int64_t)q * a.H : nullptr, a.H, ring_all,
                                                     (lds_f32 *)s_w, (lds_f32 *)s_b);
    auto clamp_page = [&](int page) { return page < 0 ? 0 : (page < a.num_pages ? page : a.num_pages - 1); };
    // Scalar loads (constant address space): waited on with lgkmcnt.
    const int b = clamp_index(((const_i32_t *)a.qseq)[q], a.batch);
    int n = GATHER ? min(((const_i32_t *)a.cand_count)[q], (int)a.cand_ld)
                   : valid_rows(((const_i32_t *)a.qpos)[q], ((const_i32_t *)a.seq_lens)[b]);
    n = (int)min64(n, a.max_rows);
    const u16 *pool = (const u16 *)a.pool;
    lds_u8 *const ring = (lds_u8 *)ring_raw + wv * NB * CHUNK;
    int tile_page = 0;
    if constexpr (!GATHER) {
        wait_vmcnt_upto(staged); // the page ids have landed (vector loads complete in issue order)
        if (b == b_guess) {
            tile_page = ((const __attribute__((address_space(3))) int32_t *)s_pg)[wv * 64 + lane];
        } else if (lane < nt_max) {
            tile_page = a.bt[(int64_t)b * a.max_pages + (tile_row0(lane) >> 6)];
        }
        tile_page = clamp_page(tile_page);
    }

    if constexpr (GATHER) {
        // Physical rows of every tile of this wave, resolved once up front
        // (candidate slots past the count read slot cand_ld-1; positions and
        // pages are clamped into the cache).
        // Two phases, so that the loads of each phase are in flight
        // together: one round trip for the candidates, one for the pages.
        const int64_t max_pos = (int64_t)a.max_pages * kPage - 1;
        int pos[kGatherTiles], page[kGatherTiles];
#pragma unroll
        for (int i = 0; i < kGatherTiles; ++i) {
            pos[i] = 0;
            if (i < nt_max) {
                int64_t j = tile_row0(i) + (lane & 31);
                j = j < a.cand_ld ? j : a.cand_ld - 1;
                pos[i] = a.cand[(int64_t)q * a.cand_ld + j];
            }
        }
        if (b == b_guess && a.max_pages <= kGatherBtLds) { // uniform over the workgroup
            // this wave's candidates have landed, and with them (vector loads
            // complete in issue order) its part of the row; the barrier waits
            // for the other waves' parts
            wg_barrier();
#pragma unroll
            for (int i = 0; i < kGatherTiles; ++i) {
                pos[i] = pos[i] < 0 ? 0 : (pos[i] > max_pos ? (int)max_pos : pos[i]);
                page[i] = i < nt_max ? ((const __attribute__((address_space(3))) int32_t *)s_bt)[pos[i] >> 6] : 0;
            }
        } else {
#pragma unroll
            for (int i = 0; i < kGatherTiles; ++i) {
                pos[i] = pos[i] < 0 ? 0 : (pos[i] > max_pos ? (int)max_pos : pos[i]);
                page[i] = 0;
                if (i < nt_max) page[i] = a.bt[(int64_t)b * a.max_pages + (pos[i] >> 6)];
            }
        }
#pragma unroll
        for (int i = 0; i < kGatherTiles; ++i)
            if (i < nt_max && lane < 32)
                s_row[(wv * kGatherTiles + i) * kTile + lane] = clamp_page(page[i]) * kPage + (pos[i] & 63);
        wait_lds();
    }
    // per-lane byte offsets of the DMA sources inside a chunk (contiguous mode)
    uint32_t src_off[NIC];
#pragma unroll
    for (int j = 0; j < NIC; ++j) {
        const int p = j * 64 + lane;
        const int nr = p / CH, cs = p % CH;
        src_off[j] = (uint32_t)((nr * R + (cs ^ (nr % CH)) * 8) * 2);
    }
    auto issue = [&](int c) {
        const int i = c / CPT;
        lds_u8 *buf = ring + (c % NB) * CHUNK;
        if constexpr (GATHER) {
            const __attribute__((address_space(3))) int32_t *rows =
                (const __attribute__((address_space(3))) int32_t *)s_row + (wv * kGatherTiles + i) * kTile;
            issue_rows<R, CH, NIC, NT>(pool, [&](int nr) { return (int64_t)rows[nr] * R; }, (c % CPT) * WC, buf, 0,
                                       NIC);
        } else {
            const int64_t t0 = tile_row0(i);
            const int page = __builtin_amdgcn_readlane(tile_page, i);
            const u16 *gbase = pool + ((int64_t)page * kPage + (t0 & 63)) * R + (c % CPT) * WC;
#pragma unroll
            for (int j = 0; j < NIC; ++j) dma16s<NT>(gbase, src_off[j], buf + j * 1024);
        }
    };
    const int npro = min(NB - 1, CPT * nt_max);
    for (int c = 0; c < npro; ++c) issue(c);

    if (a.hist && blockIdx.x == 0 && threadIdx.x == 0) {
        a.hist[(int64_t)q * kHistStride + kSlotN] = n;
        if (a.flt.filter_path) zero_filter_counters(a.hist + (int64_t)q * kHistStride);
    }
    if (row0 >= n) {
        wait_vmcnt<0>(); // no LDS write may land after the workgroup has left
        return;
    }
    if (a.hist) hist_zero(s_hist, 256, threadIdx.x);
    int nt = 0;
    if (first < n) nt = (int)min64(tiles_per_wave, (n - first + 4 * kTile - 1) / (4 * kTile));
    const int nchunks = CPT * nt; // <= CPT * nt_max: chunks issued above past it are waited for, never used
    // the query's rows and weights were issued before the chunks: they have
    // landed once at most the chunks are outstanding
    wait_after<NIC, NB - 1>(npro);
    wg_barrier(); // every wave's part of the query is in LDS (and the histogram is cleared)
    QueryRegs<R, HB> qr;
    qr.template from_lds<NB, CHUNK>(ring_all, (const lds_f32 *)s_w, (const lds_f32 *)s_b, a.bias != nullptr, a.H);
    wait_lds();
    wg_barrier(); // no wave overwrites a staging slot before every wave has read it

    __attribute__((address_space(3))) float *const outw =
        (__attribute__((address_space(3))) float *)s_out + wv * kTile;
    f32x16 acc[HB];
    // LDS offsets of this lane's B fragments inside a chunk, one per k-step
    uint32_t rd_off[KSH];
    {
        const int nr = lane & 31, g = lane >> 5;
#pragma unroll
        for (int s = 0; s < KSH; ++s) rd_off[s] = (uint32_t)((nr * CH + ((2 * s + g) ^ (nr % CH))) * 16);
    }
    // chunk c of the stream; its ring slot and its place in the tile are
    // compile-time constants (the loop runs UN chunks per round)
    constexpr int UN = NB % CPT == 0 ? NB : NB * CPT;
    auto chunk = [&](auto Uc, int c) {
        constexpr int U = decltype(Uc)::value;
        constexpr int SL = U % NB, PART = U % CPT;
        if (c + NB - 1 < nchunks) {
            wait_lds(); // this wave's reads of that buffer (chunk c-1) are complete
            issue(c + NB - 1);
        }
        wait_after<NIC, NB - 1>(min(NB - 1, nchunks - 1 - c));
        LI_PHASE_FIRST_IF(c == 0);
        const lds_u8 *buf = ring + SL * CHUNK;
        // a tile's accumulators start from the heads' biases, or (no bias)
        // its first step adds to a constant zero
        if constexpr (PART == 0 && BIAS) {
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) acc[hb] = qr.b[hb];
        }
#pragma unroll
        for (int s = 0; s < KSH; ++s) {
            const bf16x8 bfr = *(const lds_bf16x8 *)(buf + rd_off[s]);
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {
                const f32x16 zero = {};
                acc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qr.a[hb][PART * KSH + s], bfr,
                                                                  !BIAS && PART == 0 && s == 0 ? zero : acc[hb], 0,
                                                                  0, 0);
            }
        }
        if constexpr (PART == CPT - 1) {
            const float p = epilogue<HB>(acc, qr.w);
            const int i = c / CPT;
            if (lane < 32 && tile_row0(i) + lane < n)
                outw[i * 4 * kTile + lane] = p; // workgroup-local row (i * 4 + wv) * 32 + lane
        }
    };
#pragma unroll 1
    for (int c0 = 0; c0 < nchunks; c0 += UN)
        static_for<UN>([&](auto Uc) {
            const int c = c0 + decltype(Uc)::value;
            if (c < nchunks) chunk(Uc, c);
        });
    wait_vmcnt<0>(); // chunks issued ahead of the row count and never used
    LI_PHASE_LOOP;
    __syncthreads(); // every wave's scores are in LDS
    LI_PHASE_SYNC;
    // The scores leave in one pass over the workgroup's rows, which also
    // counts their first radix digit (kept out of the stream above), and
    // the fused filter pass follows when asked for.
    const int rows = (int)min64(4 * (int64_t)tiles_per_wave * kTile, n - row0);
    score_tail(a, q, row0, rows, n, (const lds_f32 *)s_out, s_hist, (FilterLds *)ring_raw);
    LI_PHASE_STORE(g_phase_bf16, wv, lane);
}

// ---------------------------------------------------------------------------
// Decode, register-staged variant: the MFMA B fragments are loaded straight
// from HBM into VGPRs (lane l reads 16 bytes of tile row l % 32 per k-step),
// DEPTH tiles deep per wave.  The VGPR file (512 KiB per CU) holds far more
// bytes in flight than the 160 KiB of LDS, which is what an HBM-bound
// stream needs; LDS keeps only the histogram (and the gather row table).
// ---------------------------------------------------------------------------
template <int R, int HB, bool GATHER, int DEPTH>
__global__ __launch_bounds__(256) void k_score_decode_vr(ScoreArgs a, int tiles_per_wave)
{
    constexpr int KS = R / 16;
    constexpr int QT_BYTES = HB * 32 * R * 2; // absorbed query, heads padded to the MFMA tile
    __shared__ __attribute__((aligned(1024))) uint8_t s_qt_raw[QT_BYTES];
    __shared__ int32_t s_row[GATHER ? 4 * kGatherTiles * kTile : 1];
    __shared__ uint32_t s_hist[kHistBins];
    __shared__ float s_out[4][kVrMaxTiles * kTile]; // scores, written out after the stream
    __shared__ float s_w[64];                       // head weights, zero past H
    __shared__ float s_b[64];                       // heads' decoder biases, zero past H (or without)

    const int q = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int b = clamp_index(a.qseq[q], a.batch);
    int n = GATHER ? min(a.cand_count[q], (int)a.cand_ld) : valid_rows(a.qpos[q], a.seq_lens[b]);
    n = (int)min64(n, a.max_rows);
    if (a.hist && blockIdx.x == 0 && threadIdx.x == 0) {
        a.hist[(int64_t)q * kHistStride + kSlotN] = n;
        if (a.flt.filter_path) zero_filter_counters(a.hist + (int64_t)q * kHistStride);
    }
    const int64_t row0 = (int64_t)blockIdx.x * 4 * tiles_per_wave * kTile;
    if (row0 >= n) return;
    if (a.hist) hist_zero(s_hist, 256, threadIdx.x);
    const int64_t first = row0 + (int64_t)wv * kTile;
    int nt = 0;
    if (first < n) nt = (int)min64(tiles_per_wave, (n - first + 4 * kTile - 1) / (4 * kTile));

    const u16 *pool = (const u16 *)a.pool;
    const_i32_t *bt = (const_i32_t *)(a.bt + (int64_t)b * a.max_pages);
    auto tile_row0 = [&](int i) -> int64_t { return first + (int64_t)i * 4 * kTile; };
    const int nr = lane & 31;
    if constexpr (GATHER) {
        for (int i = 0; i < nt; ++i) {
            int64_t j = tile_row0(i) + nr;
            j = j < n ? j : n - 1;
            const int pos = clamp_index(a.cand[(int64_t)q * a.cand_ld + j], a.max_pages * kPage);
            const int page = clamp_index(a.bt[(int64_t)b * a.max_pages + (pos >> 6)], a.num_pages);
            if (lane < 32) s_row[(wv * kGatherTiles + i) * kTile + lane] = page * kPage + (pos & 63);
        }
        wait_lds();
    }

    // this lane's row of tile i (rows past n read row n-1), first element of its k-half
    auto lane_ptr = [&](int i) -> const u16 * {
        int64_t off;
        if constexpr (GATHER) {
            off = (int64_t)s_row[(wv * kGatherTiles + i) * kTile + nr] * R;
        } else {
            const int64_t t0 = tile_row0(i);
            int64_t j = nr;
            if (t0 + j >= n) j = n - 1 - t0; // stay inside the sequence's last page
            off = ((int64_t)clamp_index(bt[t0 >> 6], a.num_pages) * kPage + (t0 & 63) + j) * R;
        }
        return pool + off + (lane >> 5) * 8;
    };
    bf16x8 bf[DEPTH][KS];
    auto load = [&](bf16x8(&dst)[KS], int i) {
        const u16 *p = lane_ptr(i);
#pragma unroll
        for (int s = 0; s < KS; ++s) dst[s] = *(const bf16x8 *)(p + s * 16);
    };

    // Prologue: this wave's quarter of the absorbed query and the head
    // weights go HBM/L2 -> VGPR -> LDS (plain loads: an LDS DMA or a weight
    // held in a VMEM-loaded register makes the compiler drain every load
    // inside the stream loop), then the first DEPTH tiles are issued.  The
    // loop is entered with exactly DEPTH tiles of loads pending, the same
    // state its back edge carries, so every wait in it stays exact.
    constexpr int QCH = (QT_BYTES / 1024 + 3) / 4; // 1 KiB pieces of the query per wave
    u32x4 qv[QCH];
    const int qbytes = a.H * R * 2;
    {
        const uint8_t *src = (const uint8_t *)((const u16 *)a.qt + (int64_t)q * a.H * R);
#pragma unroll
        for (int c = 0; c < QCH; ++c) {
            int off = (c * 4 + wv) * 1024 + lane * 16;
            off = off < qbytes ? off : qbytes - 16;
            qv[c] = *(const u32x4 *)(src + off);
        }
    }
    const float wv_lane = a.w[(int64_t)q * a.H + (lane < a.H ? lane : a.H - 1)];
    const float bv_lane = a.bias ? a.bias[(int64_t)q * a.H + (lane < a.H ? lane : a.H - 1)] : 0.0f;
    if (nt > 0) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) load(bf[d], d < nt ? d : nt - 1);
    }
#pragma unroll
    for (int c = 0; c < QCH; ++c) {
        const int off = (c * 4 + wv) * 1024 + lane * 16;
        if (off < qbytes) *(lds_u32x4 *)((lds_u8 *)s_qt_raw + off) = qv[c];
    }
    if (wv == 0) s_w[lane] = lane < a.H ? wv_lane : 0.0f;
    if (wv == 1) s_b[lane] = lane < a.H ? bv_lane : 0.0f;
    wg_barrier(); // every wave's part of the query is in LDS; histogram cleared
    QueryRegs<R, HB> qr;
    {
        const int h = lane & 31;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                if (hb * 32 + h < a.H) {
                    qr.a[hb][s] = *(lds_bf16x8 *)((lds_u8 *)s_qt_raw +
                                                   ((hb * 32 + h) * R + s * 16 + (lane >> 5) * 8) * 2);
                } else {
                    bf16x8 z = {};
                    qr.a[hb][s] = z;
                }
            }
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int hh = hb * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                qr.w[hb][r] = ((const lds_f32 *)s_w)[hh];
                qr.b[hb][r] = ((const lds_f32 *)s_b)[hh];
            }
    }

    float *out = a.out + (int64_t)q * a.out_ld;
    auto compute = [&](const bf16x8(&src)[KS]) {
        f32x16 acc[HB];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) acc[hb] = qr.b[hb];
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int hb = 0; hb < HB; ++hb)
                acc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qr.a[hb][s], src[s], acc[hb], 0, 0, 0);
        return epilogue<HB>(acc, qr.w);
    };
    // Scores wait in LDS until the stream is done: a global store among the
    // loads would make every wait in the loop a full drain.
    auto store = [&](float p, int i) {
        const int64_t j = tile_row0(i) + nr;
        if (lane < 32) {
            s_out[wv][i * kTile + lane] = p;
            if (j < n && a.hist) atomicAdd(&s_hist[score_key(p) >> kDigit0Shift], 1u);
        }
    };
    if (nt > 0) {
        int i0 = 0;
        // Steady state: every slot is refilled right after use, unconditionally,
        // so each wait is for exactly the oldest tile's loads.
        for (; i0 + 2 * DEPTH <= nt; i0 += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const float p = compute(bf[d]);
                load(bf[d], i0 + d + DEPTH);
                store(p, i0 + d);
            }
        }
        // Tail: the last (< 2 DEPTH) tiles.
        for (; i0 < nt; i0 += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int i = i0 + d;
                if (i < nt) {
                    const float p = compute(bf[d]);
                    if (i + DEPTH < nt) load(bf[d], i + DEPTH);
                    store(p, i);
                }
            }
        }
    }
    // this wave's scores: two tiles per store instruction
    wait_lds();
    for (int i = lane >> 5; i < nt; i += 2) {
        const int64_t j = tile_row0(i) + nr;
        if (j < n) out[j] = s_out[wv][i * kTile + nr];
    }
    if (a.hist) {
        __syncthreads();
        hist_flush(s_hist, a.hist + (int64_t)q * kHistStride, 256, threadIdx.x);
    }
}

// ---------------------------------------------------------------------------
// Prefill: many queries per sequence.  Workgroup = 4 consecutive queries,
// one per wave; the 4 waves share every latent tile (one DMA per tile,
// split across the waves) through an NBUF-deep LDS ring, one barrier per
// tile.  The page ids of a split's tiles are staged in LDS first, so no
// dependent global load sits in the stream.  Queries of a workgroup that
// sit in different sequences are served in separate passes.  The LDS
// footprint (ring + page ids) leaves room for two workgroups per CU, so a
// second wave on each SIMD covers barriers and epilogues; the first radix
// digit is counted by the selection pass instead of here.
// ---------------------------------------------------------------------------
template <int R, int HB, int NBUF, int QW, int TPB, bool BIAS>
__global__ __launch_bounds__(64 * QW) __attribute__((amdgpu_waves_per_eu(2))) void k_score_prefill(
    ScoreArgs a, int tiles_per_split)
{
    constexpr int TILE_BYTES = kTile * R * 2;
    constexpr int CH = R / 8;
    constexpr int NI = R / 16;
    constexpr int NIW = NI / QW;
    constexpr int NT = 64 * QW;
    static_assert(NIW >= 1 && NIW * QW == NI, "tile must split over the waves");
    static_assert(NBUF >= 3, "ring depth");
    __shared__ __attribute__((aligned(1024))) uint8_t ring_raw[NBUF * TILE_BYTES];
    __shared__ int32_t s_page_raw[kPrefillMaxTiles / 2 + 2];
    lds_u8 *ring = (lds_u8 *)ring_raw;
    lds_i32 *s_page = (lds_i32 *)s_page_raw;

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int qbase = blockIdx.x * QW;
    const_i32_t *qseq = (const_i32_t *)a.qseq;
    const_i32_t *qpos = (const_i32_t *)a.qpos;
    const_i32_t *slen = (const_i32_t *)a.seq_lens;
    int sb[QW], sn[QW];
#pragma unroll
    for (int u = 0; u < QW; ++u) {
        const int qq = qbase + u;
        sb[u] = qq < a.Q ? clamp_index(qseq[qq], a.batch) : -1;
        sn[u] = qq < a.Q ? (int)min64(valid_rows(qpos[qq], slen[sb[u]]), a.max_rows) : 0;
    }
    const int q = qbase + wv;
    int my_b = -1, my_n = 0;
#pragma unroll
    for (int u = 0; u < QW; ++u)
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
    // with a bias, one MFMA per head block starts each tile's accumulators
    bf16x8 ab[HB], bones;
    if constexpr (BIAS) bias_operands<HB>(a.bias + (int64_t)(q < a.Q ? q : 0) * a.H, a.H, q < a.Q, ab, bones);
    float *out = a.out + (int64_t)(q < a.Q ? q : 0) * a.out_ld;
    const u16 *pool = (const u16 *)a.pool;

#pragma unroll 1
    for (int u = 0; u < QW; ++u) {
        const int b = sb[u];
        bool skip = b < 0;
        int nmax = 0;
#pragma unroll
        for (int v = 0; v < QW; ++v) {
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
        // page ids of rows [ts*32, te*32): pages ts/2 .. (te-1)/2
        const int p0 = ts >> 1;
        const int np = ((te - 1) >> 1) - p0 + 1;
        __syncthreads(); // the previous pass is done with the ring and the page ids
        for (int pi = threadIdx.x; pi < np; pi += NT)
            s_page[pi] = clamp_index(a.bt[(int64_t)b * a.max_pages + p0 + pi], a.num_pages);
        __syncthreads();
        auto page_of = [&](int i) { return s_page[((ts + i) >> 1) - p0]; };
        auto issue = [&](int i, int page) {
            const int64_t base = ((int64_t)page * kPage + ((ts + i) & 1) * kTile) * R;
            issue_rows<R, CH, NIW>(pool, [&](int nr) { return base + (int64_t)nr * R; }, 0,
                                   ring + (i % NBUF) * TILE_BYTES, wv * NIW, NIW);
        };
        // Tiles move in groups of TPB: one wait and one barrier per group.
        // Tile i sits in slot i % NBUF; group g+NG-1 refills group g-1's slots.
        constexpr int NG = NBUF / TPB;
        static_assert(NG * TPB == NBUF && NG >= 2, "ring groups");
        const int ngr = (nt + TPB - 1) / TPB;
        for (int gq = 0; gq < NG - 1 && gq < ngr; ++gq)
#pragma unroll
            for (int t = 0; t < TPB; ++t)
                if (gq * TPB + t < nt) issue(gq * TPB + t, page_of(gq * TPB + t));
#pragma unroll 1
        for (int gq = 0; gq < ngr; ++gq) {
            const int gnext = gq + NG - 1;
            int pnext[TPB];
#pragma unroll
            for (int t = 0; t < TPB; ++t) // read before the barrier
                pnext[t] = gnext * TPB + t < nt ? page_of(gnext * TPB + t) : 0;
            // this group landed (this wave's parts); the tiles issued after it may still fly
            const int after = min((gq + NG - 1) * TPB, nt) - (gq + 1) * TPB;
            wait_after<NIW, (NG - 2) * TPB < 1 ? 1 : (NG - 2) * TPB>(after > 0 ? after : 0);
            wg_barrier(); // every part of the group landed; every wave is done with the previous group
#pragma unroll
            for (int t = 0; t < TPB; ++t)
                if (gnext < ngr && gnext * TPB + t < nt) issue(gnext * TPB + t, pnext[t]);
            if (active) {
#pragma unroll
                for (int t = 0; t < TPB; ++t) {
                    const int i = gq * TPB + t;
                    if (i >= nt) break;
                    // the chains start from the heads' biases or a constant zero
                    f32x16 acc[HB];
                    if constexpr (BIAS) {
#pragma unroll
                        for (int hb = 0; hb < HB; ++hb) {
                            const f32x16 zero = {};
                            acc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab[hb], bones, zero, 0, 0, 0);
                        }
                    }
                    mfma_tile_prefetch<R, HB, CH, 4, !BIAS>(ring + (i % NBUF) * TILE_BYTES, qr, acc);
                    const float p = epilogue<HB>(acc, qr.w);
                    const int j = (ts + i) * kTile + lane;
                    if (lane < 32 && j < my_n) out[j] = p;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 latent (any r <= 256): plain VALU dot products, one row per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_score_f32(ScoreArgs a, int R, int rows_per_wg)
{
    __shared__ float sq[64 * 256];
    __shared__ float sw[64];
    __shared__ float sb[64];
    __shared__ uint32_t s_hist[kHistBins];
    const int q = blockIdx.y;
    const int b = clamp_index(a.qseq[q], a.batch);
    int n = a.cand ? min(a.cand_count[q], (int)a.cand_ld) : valid_rows(a.qpos[q], a.seq_lens[b]);
    n = (int)min64(n, a.max_rows);
    if (a.hist && blockIdx.x == 0 && threadIdx.x == 0) {
        a.hist[(int64_t)q * kHistStride + kSlotN] = n;
        if (a.flt.filter_path) zero_filter_counters(a.hist + (int64_t)q * kHistStride);
    }
    const int64_t row0 = (int64_t)blockIdx.x * rows_per_wg;
    if (row0 >= n) return;
    const int64_t row1 = min64(row0 + rows_per_wg, n);
    const float *qt = (const float *)a.qt + (int64_t)q * a.H * R;
    for (int i = threadIdx.x; i < a.H * R; i += 256) sq[i] = qt[i];
    for (int i = threadIdx.x; i < a.H; i += 256) {
        sw[i] = a.w[(int64_t)q * a.H + i];
        sb[i] = a.bias ? a.bias[(int64_t)q * a.H + i] : 0.0f;
    }
    if (a.hist) hist_zero(s_hist, 256, threadIdx.x);
    __syncthreads();
    for (int64_t j = row0 + threadIdx.x; j < row1; j += 256) {
        const int pos = a.cand ? clamp_index(a.cand[(int64_t)q * a.cand_ld + j], a.max_pages * kPage) : (int)j;
        const int page = clamp_index(a.bt[(int64_t)b * a.max_pages + (pos >> 6)], a.num_pages);
        const float *row = (const float *)a.pool + ((int64_t)page * kPage + (pos & 63)) * R;
        float sc = 0.0f;
        for (int h = 0; h < a.H; ++h) {
            float dot = 0.0f;
            for (int t = 0; t < R; ++t) dot = fmaf(sq[h * R + t], row[t], dot);
            sc = fmaf(sw[h], fmaxf(dot + sb[h], 0.0f), sc);
        }
        a.out[(int64_t)q * a.out_ld + j] = sc;
        if (a.hist) atomicAdd(&s_hist[score_key(sc) >> kDigit0Shift], 1u);
    }
    if (a.hist) {
        __syncthreads();
        hist_flush(s_hist, a.hist + (int64_t)q * kHistStride, 256, threadIdx.x);
    }
}

// Decode kernel choice.  Measured on MI355X: the register-staged kernel is
// faster for r = 64 over contiguous prefixes (its deeper in-flight window
// matters most when each tile is small); the LDS ring is faster from r = 128
// (whole-tile chunks there) and for gathered rows.  LI_DECODE_PATH=lds|vgpr
// overrides (read once).
int decode_path_override()
{
    static const int path = [] {
        const char *e = getenv("LI_DECODE_PATH");
        if (e && strcmp(e, "lds") == 0) return 0;
        if (e && strcmp(e, "vgpr") == 0) return 1;
        return -1;
    }();
    return path;
}

bool use_vgpr_decode(int r, bool gather)
{
    const int o = decode_path_override();
    if (o >= 0) return o == 1;
    return r <= 64 && !gather;
}

template <int R, int HB>
hipError_t launch_bf16(const ScoreArgs &a, bool prefill, int64_t max_rows, hipStream_t s, bool *filtered)
{
    const int64_t tiles = (max_rows + kTile - 1) / kTile;
    if (prefill) {
        constexpr int NBUF = R == 256 ? 4 : 6;
        constexpr int QW = 4;
        constexpr int TPB = 1; // tiles per barrier
        const int qblocks = (a.Q + QW - 1) / QW;
        int64_t splits = 1;
        if (qblocks < 512) splits = std::min<int64_t>((512 + qblocks - 1) / qblocks, tiles);
        if (splits < 1) splits = 1;
        int64_t tps = (tiles + splits - 1) / splits;
        if (tps > kPrefillMaxTiles) tps = kPrefillMaxTiles;
        splits = (tiles + tps - 1) / tps;
        if (a.bias)
            return launch_kernel(k_score_prefill<R, HB, NBUF, QW, TPB, true>, dim3(qblocks, (unsigned)splits),
                                 dim3(64 * QW), 0, s, a, (int)tps);
        return launch_kernel(k_score_prefill<R, HB, NBUF, QW, TPB, false>, dim3(qblocks, (unsigned)splits),
                             dim3(64 * QW), 0, s, a, (int)tps);
    }
    // decode: about one round of one workgroup per CU
    const int64_t want_wgs = 256;
    const int64_t per_q = (want_wgs + a.Q - 1) / a.Q;
    int64_t tpw = (tiles + 4 * per_q - 1) / (4 * per_q);
    if (tpw < 1) tpw = 1;
    if (a.cand && tpw > kGatherTiles) tpw = kGatherTiles;
    int64_t wgs = (tiles + 4 * tpw - 1) / (4 * tpw);
    if (use_vgpr_decode(R, a.cand != nullptr)) {
        constexpr int DEPTH = R == 256 ? 3 : (R == 128 ? 5 : 8);
        if (tpw > kVrMaxTiles) {
            tpw = kVrMaxTiles;
            wgs = (tiles + 4 * tpw - 1) / (4 * tpw);
        }
        if (a.cand)
            return launch_kernel(k_score_decode_vr<R, HB, true, DEPTH>, dim3((unsigned)wgs, a.Q), dim3(256), 0, s, a,
                                 (int)tpw);
        return launch_kernel(k_score_decode_vr<R, HB, false, DEPTH>, dim3((unsigned)wgs, a.Q), dim3(256), 0, s, a,
                             (int)tpw);
    }
    if (!a.cand && tpw > kMaxTilesPerWave) {
        tpw = kMaxTilesPerWave; // one page id per lane of the wave
        wgs = (tiles + 4 * tpw - 1) / (4 * tpw);
    }
    // chunk ring: 96 KiB next to the histogram and the staged scores
    constexpr int CPT = R == 256 ? 2 : 1;
    constexpr int NB = R == 64 ? 6 : 3;
    // the filter pass rides along when every workgroup of the grid is resident
    ScoreArgs b = a;
    b.flt.on = a.flt.on && !a.cand && a.hist && fused_filter_fits(wgs, a.Q);
    if (filtered) *filtered = b.flt.on;
    auto go = [&](auto BIASc) {
        constexpr bool BI = decltype(BIASc)::value;
        const dim3 grid((unsigned)wgs, b.Q);
        if (b.cand) return launch_kernel(k_score_decode<R, HB, true, NB, CPT, false, BI>, grid, dim3(256), 0, s, b, (int)tpw);
        if (b.stream_nt)
            return launch_kernel(k_score_decode<R, HB, false, NB, CPT, true, BI>, grid, dim3(256), 0, s, b, (int)tpw);
        return launch_kernel(k_score_decode<R, HB, false, NB, CPT, false, BI>, grid, dim3(256), 0, s, b, (int)tpw);
    };
    return b.bias ? go(std::true_type{}) : go(std::false_type{});
}

template <int R>
hipError_t launch_r(const ScoreArgs &a, bool prefill, int64_t max_rows, hipStream_t s, bool *filtered)
{
    if (a.H <= 32) return launch_bf16<R, 1>(a, prefill, max_rows, s, filtered);
    return launch_bf16<R, 2>(a, prefill, max_rows, s, filtered);
}

// Candidate scores from scores kept by position.
__global__ __launch_bounds__(256) void k_gather_scores(const float *S, int64_t ld, const int32_t *cand,
                                                       const int32_t *cand_count, int64_t M, float *out)
{
    const int q = blockIdx.y;
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n = min64(max(cand_count[q], 0), M);
    if (j >= n) return;
    int64_t c = cand[(int64_t)q * M + j];
    c = c < 0 ? 0 : (c < ld ? c : ld - 1);
    out[(int64_t)q * M + j] = S[(int64_t)q * ld + c];
}

} // namespace

#ifdef LI_PHASE_PROBE
hipError_t phase_records_bf16(void **dev) { return hipGetSymbolAddress(dev, HIP_SYMBOL(g_phase_bf16)); }
#else
hipError_t phase_records_bf16(void **dev)
{
    *dev = nullptr;
    return hipErrorNotSupported;
}
#endif

hipError_t launch_gather_scores(const float *S, int64_t ld, const int32_t *cand, const int32_t *cand_count, int64_t M,
                                float *out, int32_t Q, hipStream_t s)
{
    if (Q <= 0 || M <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_gather_scores, dim3((unsigned)((M + 255) / 256), Q), dim3(256), 0, s, S, ld, cand, cand_count,
                       M, out);
    return hipGetLastError();
}

int device_cu_count()
{
    static int cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cus[dev] <= 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cus[dev] = v;
    }
    return cus[dev];
}

bool fused_filter_fits(int64_t wgs_per_query, int64_t Q)
{
    // one decode scoring workgroup per CU fits (its LDS allows no more), so
    // a grid of at most one workgroup per CU is resident at once
    return wgs_per_query * Q <= device_cu_count();
}

hipError_t launch_score(const ScoreArgs &a, int r, bool bf16, bool many_queries_per_seq, int64_t max_rows,
                        hipStream_t s, bool *filtered)
{
    if (filtered) *filtered = false;
    if (a.Q <= 0 || max_rows <= 0) return hipSuccess;
    const bool prefill = many_queries_per_seq && a.cand == nullptr;
    if (!bf16) {
        const int64_t wgs = std::min<int64_t>((max_rows + 255) / 256, 1024);
        const int64_t per = ((max_rows + wgs - 1) / wgs + 255) / 256 * 256;
        return launch_kernel(k_score_f32, dim3((unsigned)((max_rows + per - 1) / per), a.Q), dim3(256), 0, s, a, r,
                             (int)per);
    }
    switch (r) {
    case 64: return launch_r<64>(a, prefill, max_rows, s, filtered);
    case 128: return launch_r<128>(a, prefill, max_rows, s, filtered);
    case 256: return launch_r<256>(a, prefill, max_rows, s, filtered);
    default: return hipErrorInvalidValue;
    }
}

} // namespace li

// Segmented FP8 latent cache, FP8 queries and FP8 MFMA scoring (gfx950).
//
// LatentIndex (paperlayer.ai summary of arXiv:2610.04635), §B.2: the
// indexer runs in segmented FP8; §A.2: the decoder is absorbed into the
// query before the Hadamard rotation, so both operands are rotated ahead of
// quantization and their dot products are unchanged by it.  The pages fix no
// format; the one used here:
//   - each 128-element segment of a latent row or of an absorbed query head
//     is rotated by the orthonormal Walsh-Hadamard transform (fp32
//     butterflies with strides 1, 2, ..., 64, then a multiply by the fp32
//     value of 1/sqrt(128));
//   - the segment gets a power-of-two scale 2^e, e the smallest integer with
//     amax * 2^-e <= 448 (clamped to [-120, 120]);
//   - every element is stored as the OCP FP8 E4M3 code of x * 2^-e (round to
//     nearest even, saturating at 448).
// Power-of-two scales make the scaling exact and map onto the E8M0 block
// scales of v_mfma_scale_f32_32x32x64_f8f6f4, which applies them to each
// lane's block of 32 codes inside the MFMA: the score is
//   sum_h w_h max(0, sum_seg sq[h][seg] sc[j][seg] sum_{t in seg} q8[h][t] c8[j][t])
// with exact products and fp32 accumulation.
//
// Layouts.  Latent: codes [page][64][r] bytes beside scales [page][64][r/128]
// fp32 (powers of two).  Query: one buffer, codes [Q][H][r] bytes then, at
// byte offset li_fp8_query_scale_offset(Q, H, r), scales [Q][H][r/128] fp32.
#include "li_device.hpp"
#include "li_internal.hpp"
#include "li_probe.hpp"
#include "li_tail.hpp"
#include "li_timing.hpp"

#include <algorithm>

namespace li {

#ifdef LI_PHASE_PROBE
__device__ uint64_t g_phase_fp8[kProbeWaves * kProbeWords]; // phase records (instrumented build only)
#endif
namespace {

constexpr int kSeg = 128;               // elements per quantization segment
constexpr int kGatherTilesF8 = 16;      // max tiles per wave in gather mode
constexpr int kMaxTilesPerWaveF8 = 64;  // max tiles per wave in contiguous mode (their scores stay in LDS)

// 2^k as an fp32 (k in [-126, 127]).
__device__ __forceinline__ float exp2i(int k) { return __uint_as_float((uint32_t)(k + 127) << 23); }

// Nearest E4M3 code (ties to the even mantissa), saturating at 448.  The
// steps follow the format definition: magnitudes below 2^-6 go in steps of
// 2^-9 (code = step count; 8 steps is the smallest normal, code 8); above,
// three mantissa bits under the binade's exponent.
__device__ __forceinline__ uint32_t e4m3_encode(float v)
{
    const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
    const float a = fabsf(v);
    if (!(a > 0.0f)) return sign;
    if (a >= 448.0f) return sign | 0x7Eu;
    const int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127; // floor(log2 a); fp32 subnormals land below -6
    if (e < -6) return sign | (uint32_t)rintf(a * 512.0f);
    int m = (int)rintf(a * exp2i(3 - e)); // 8 .. 16
    int ee = e;
    if (m == 16) {
        m = 8;
        ee += 1;
    }
    return sign | (uint32_t)(((ee + 7) << 3) | (m - 8));
}

// Smallest e with amax * 2^-e <= 448 (0 for amax == 0), clamped to [-120, 120].
__device__ __forceinline__ int pow2_exponent(float amax)
{
    if (!(amax > 0.0f)) return 0;
    int E;
    const float f = frexpf(amax, &E); // amax = (2f) 2^(E-1), 2f in [1, 2)
    int e = (2.0f * f <= 1.75f) ? E - 9 : E - 8;
    return e < -120 ? -120 : (e > 120 ? 120 : e);
}

// v from lane (l ^ d) of the same 32-lane half (d < 32): ds_swizzle in
// bit-mask mode (and 0x1F, or 0, xor d), no LDS access.
template <int D>
__device__ __forceinline__ float xor32(float v)
{
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (D << 10) | 0x1F));
}

// Rotate and quantize NR 128-element segments, each held by the 32 lanes of
// a half-wave, four consecutive elements per lane (lane l32 holds elements
// 4*l32 .. 4*l32+3 of each).  Returns the four codes of each segment packed
// little-endian; e[k] receives segment k's scale exponent.  The butterflies
// run in the order of the definition (strides 1, 2 inside the lane, then
// 4 .. 64 across lanes), each output being lower + upper or lower - upper,
// so the fp32 results are the definition's to the bit.  The NR segments are
// independent chains, interleaved to hide the cross-lane latency.
template <int D, int NR>
__device__ __forceinline__ void butterfly_stage(float (&x)[NR][4], bool upper)
{
    float p[NR][4];
#pragma unroll
    for (int k = 0; k < NR; ++k)
#pragma unroll
        for (int t = 0; t < 4; ++t) p[k][t] = xor32<D>(x[k][t]);
#pragma unroll
    for (int k = 0; k < NR; ++k)
#pragma unroll
        for (int t = 0; t < 4; ++t) x[k][t] = upper ? p[k][t] - x[k][t] : x[k][t] + p[k][t];
}

template <int D, int NR>
__device__ __forceinline__ void amax_stage(float (&m)[NR])
{
    float p[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) p[k] = xor32<D>(m[k]);
#pragma unroll
    for (int k = 0; k < NR; ++k) m[k] = fmaxf(m[k], p[k]);
}

template <int NR>
__device__ __forceinline__ void rotate_quantize(float (&x)[NR][4], int l32, int (&e)[NR], uint32_t (&codes)[NR])
{
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        {
            const float a0 = x[k][0], b0 = x[k][1], a1 = x[k][2], b1 = x[k][3];
            x[k][0] = a0 + b0;
            x[k][1] = a0 - b0;
            x[k][2] = a1 + b1;
            x[k][3] = a1 - b1;
        }
        {
            const float a0 = x[k][0], b0 = x[k][2], a1 = x[k][1], b1 = x[k][3];
            x[k][0] = a0 + b0;
            x[k][2] = a0 - b0;
            x[k][1] = a1 + b1;
            x[k][3] = a1 - b1;
        }
    }
    butterfly_stage<1>(x, (l32 & 1) != 0);
    butterfly_stage<2>(x, (l32 & 2) != 0);
    butterfly_stage<4>(x, (l32 & 4) != 0);
    butterfly_stage<8>(x, (l32 & 8) != 0);
    butterfly_stage<16>(x, (l32 & 16) != 0);
    const float kn = 0.08838834764831845f; // 1/sqrt(128)
    float amax[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        amax[k] = 0.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            x[k][t] = x[k][t] * kn;
            amax[k] = fmaxf(amax[k], fabsf(x[k][t]));
        }
    }
    amax_stage<1>(amax);
    amax_stage<2>(amax);
    amax_stage<4>(amax);
    amax_stage<8>(amax);
    amax_stage<16>(amax);
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        e[k] = pow2_exponent(amax[k]);
        const float inv = exp2i(-e[k]);
        uint32_t packed = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) packed |= e4m3_encode(x[k][t] * inv) << (8 * t);
        codes[k] = packed;
    }
}

// ---------------------------------------------------------------------------
// Append: bf16 rows [T][R] -> rotated, quantized codes and segment scales at
// their page slots.  One half-wave per (row, segment).
// ---------------------------------------------------------------------------
template <int R>
__global__ __launch_bounds__(256) void k_append_fp8(uint8_t *pool, float *scales, const int32_t *bt, PoolGeom geo,
                                                    const u16 *rows, const int32_t *seq, const int32_t *pos, int T,
                                                    const RopeArgs rope)
{
    constexpr int NSEG = R / kSeg;
    const int half = (int)((blockIdx.x * 256 + threadIdx.x) >> 5); // (row, segment) index
    const int l32 = threadIdx.x & 31;
    const int t = half / NSEG, g = half % NSEG;
    const bool live = t < T;
    const int tc = live ? t : T - 1; // lanes past the end mirror the last row and store nothing
    const uint2 raw = *(const uint2 *)(rows + (int64_t)tc * R + g * kSeg + 4 * l32);
    float x[1][4] = {{bf16_to_f32((u16)(raw.x & 0xFFFF)), bf16_to_f32((u16)(raw.x >> 16)),
                      bf16_to_f32((u16)(raw.y & 0xFFFF)), bf16_to_f32((u16)(raw.y >> 16))}};
    if (rope.F > 0) {
        // rotary source pairs among this lane's four elements: rotated in
        // fp64 at the row's position, rounded once to fp32
        const int p = pos[tc];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int j = g * (kSeg / 2) + 2 * l32 + u;
            if (j < rope.S * rope.F) {
                double re = x[0][2 * u], im = x[0][2 * u + 1];
                rope_pair(re, im, p, rope.theta[j % rope.F]);
                x[0][2 * u] = (float)re;
                x[0][2 * u + 1] = (float)im;
            }
        }
    }
    int ee[1];
    uint32_t cw[1];
    rotate_quantize<1>(x, l32, ee, cw);
    const uint32_t codes = cw[0];
    const int e = ee[0];
    if (!live) return;
    const int64_t slot = geo.slot(bt, seq[t], pos[t]);
    if (slot < 0) return; // a sequence, position or page outside the cache: the row is not written
    *(uint32_t *)(pool + slot * R + g * kSeg + 4 * l32) = codes;
    if (l32 == 0) scales[slot * NSEG + g] = exp2i(e);
}

// ---------------------------------------------------------------------------
// Absorption into an FP8 query: qt = q W_dec with every bf16 x bf16 product
// (exact in fp32) summed in fp64 and rounded once to fp32.  For bf16 inputs
// of ordinary range the fp64 sum is exact, so qt is the correctly rounded
// product whatever the summation order, and the FP8 codes do not depend on
// the tiling.  Workgroup = MB (query, head) rows x one 128-column segment:
// chunks of q (transposed) and W are staged in LDS as fp32, each thread
// holds an RT x CT tile of fp64 accumulators; the fp32 results go back
// through the same LDS and each (row, segment) is rotated and quantized by a
// half-wave.
// ---------------------------------------------------------------------------
// IDENT: no decoder (W unused, D == R): the query itself is rotated and
// quantized (a per-layer indexer's query).
constexpr int64_t kAbsorbRowMax = 1024; // rows up to which the per-row kernel is used
template <int R, int D, int MB, bool IDENT = false>
__global__ __launch_bounds__(256) void k_absorb_fp8(const u16 *q, const u16 *W, uint8_t *codes, float *qscales,
                                                    int64_t QH)
{
    static_assert(MB == 8 || MB == 32 || MB == 128, "row block");
    constexpr int NSEG = R / kSeg;
    // k per staged chunk: all of k at once for the small row blocks (few
    // rows: one load round instead of two), 64 for the prefill-sized blocks
    // (two workgroups per CU)
    constexpr int KC = MB < 128 ? (D < 128 ? D : 128) : (D < 64 ? D : 64);
    constexpr int CT = MB == 128 ? 8 : 4;    // columns per thread
    constexpr int NCG = kSeg / CT;           // column groups
    constexpr int NRG = 256 / NCG;           // row groups
    constexpr int RT = MB / NRG;             // rows per thread
    static_assert(RT >= 1 && RT * NRG == MB, "thread tile");
    constexpr int QLD = MB + 4;              // floats per staged k row of q
    constexpr int WLD = kSeg + 4;            // floats per staged k row of W
    constexpr int OLD = kSeg + 4;            // floats per staged result row
    constexpr int STAGE = KC * (QLD + WLD);
    constexpr int LDSF = STAGE > MB * OLD ? STAGE : MB * OLD;
    __shared__ __attribute__((aligned(16))) float lds[LDSF];
    float *s_q = lds;                        // [KC][QLD]
    float *s_w = lds + KC * QLD;             // [KC][WLD]
    float *s_out = lds;                      // [MB][OLD], once the sums are done
    const int tid = threadIdx.x;
    const int g = blockIdx.y;                // segment
    const int c0 = g * kSeg;
    const int64_t mb0 = (int64_t)blockIdx.x * MB;
    const int tr = tid / NCG, tc = tid % NCG;

    if constexpr (IDENT) {
        static_assert(D == R, "the identity keeps the width");
        // this segment of each row, bf16 -> fp32 (exact)
        for (int it = tid; it < MB * (kSeg / 8); it += 256) {
            const int row = it / (kSeg / 8), cc = (it % (kSeg / 8)) * 8;
            const int64_t m = mb0 + row;
            u32x4 raw = {0u, 0u, 0u, 0u};
            if (m < QH) raw = *(const u32x4 *)(q + m * R + c0 + cc);
            const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
            float *dst = s_out + row * OLD + cc;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dst[2 * i] = __uint_as_float(wd[i] << 16);
                dst[2 * i + 1] = __uint_as_float(wd[i] & 0xFFFF0000u);
            }
        }
    } else {
    double acc[RT][CT];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < CT; ++j) acc[i][j] = 0.0;

#pragma unroll 1
    for (int k0 = 0; k0 < D; k0 += KC) {
        if (k0) __syncthreads(); // every thread is done with the previous chunk
        for (int it = tid; it < MB * (KC / 8); it += 256) {
            const int row = it % MB, kk = (it / MB) * 8;
            const int64_t m = mb0 + row;
            u32x4 raw = {0u, 0u, 0u, 0u};
            if (m < QH) raw = *(const u32x4 *)(q + m * D + k0 + kk);
            const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s_q[(kk + 2 * i) * QLD + row] = __uint_as_float(wd[i] << 16);
                s_q[(kk + 2 * i + 1) * QLD + row] = __uint_as_float(wd[i] & 0xFFFF0000u);
            }
        }
        for (int it = tid; it < KC * (kSeg / 8); it += 256) {
            const int kk = it / (kSeg / 8), cc = (it % (kSeg / 8)) * 8;
            const u32x4 raw = *(const u32x4 *)(W + (int64_t)(k0 + kk) * R + c0 + cc);
            float *dst = s_w + kk * WLD + cc;
            const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dst[2 * i] = __uint_as_float(wd[i] << 16);
                dst[2 * i + 1] = __uint_as_float(wd[i] & 0xFFFF0000u);
            }
        }
        __syncthreads();
#pragma unroll 4
        for (int kk = 0; kk < KC; ++kk) {
            double a[RT], b[CT];
#pragma unroll
            for (int i = 0; i < RT; ++i) a[i] = (double)s_q[kk * QLD + tr * RT + i];
#pragma unroll
            for (int j = 0; j < CT; ++j) b[j] = (double)s_w[kk * WLD + tc * CT + j];
#pragma unroll
            for (int i = 0; i < RT; ++i)
#pragma unroll
                for (int j = 0; j < CT; ++j) acc[i][j] = __builtin_fma(a[i], b[j], acc[i][j]);
        }
    }
    __syncthreads(); // the staged chunks are no longer read: the space becomes s_out
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < CT; ++j) s_out[(tr * RT + i) * OLD + tc * CT + j] = (float)acc[i][j];
    }
    __syncthreads();
    const int lane = tid & 63, wv = tid >> 6;
    // quantization: the MB rows split over the 8 half-waves, NR rows each per pass
    constexpr int ROWS_PER_HALF = MB / 8;
    constexpr int NR = ROWS_PER_HALF < 8 ? ROWS_PER_HALF : 8;
    const int l32 = lane & 31;
    const int half = wv * 2 + (lane >> 5);
#pragma unroll 1
    for (int rr = 0; rr < ROWS_PER_HALF; rr += NR) {
        float x[NR][4];
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            const int row = (rr + k) * 8 + half;
#pragma unroll
            for (int t = 0; t < 4; ++t) x[k][t] = s_out[row * OLD + 4 * l32 + t];
        }
        int e[NR];
        uint32_t cw[NR];
        rotate_quantize<NR>(x, l32, e, cw);
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            const int64_t m = mb0 + (rr + k) * 8 + half;
            if (m < QH) {
                *(uint32_t *)(codes + m * R + c0 + 4 * l32) = cw[k];
                if (l32 == 0) qscales[m * NSEG + g] = exp2i(e[k]);
            }
        }
    }
}

// Few rows (decode): one workgroup per (query, head) row and segment, so a
// batch-1 decode step spreads over H x R/128 workgroups instead of a handful.
// Thread t owns output column t % 128 and half of k; the two fp64 partial
// sums meet in LDS (exact, as above, so the split does not change the
// result); the first wave rotates and quantizes the row segment.
// IDENT as above.
template <int R, int D, bool IDENT>
__global__ __launch_bounds__(256) void k_absorb_fp8_row(const u16 *q, const u16 *W, uint8_t *codes, float *qscales)
{
    constexpr int NSEG = R / kSeg;
    constexpr int KH = D / 2; // k per thread
    __shared__ float s_q[D];
    __shared__ double s_part[kSeg];
    __shared__ float s_out[kSeg];
    const int tid = threadIdx.x;
    const int64_t m = blockIdx.x;
    const int g = blockIdx.y;
    const int c0 = g * kSeg;
    const int c = tid & (kSeg - 1), half = tid >> 7;
    if constexpr (IDENT) {
        static_assert(D == R, "the identity keeps the width");
        if (tid < kSeg) s_out[tid] = bf16_to_f32(q[m * D + c0 + tid]);
    } else {
        for (int i = tid; i < D; i += 256) s_q[i] = bf16_to_f32(q[m * D + i]);
        float wv[KH];
#pragma unroll
        for (int kk = 0; kk < KH; ++kk) wv[kk] = bf16_to_f32(W[(int64_t)(half * KH + kk) * R + c0 + c]);
        __syncthreads();
        double acc = 0.0;
#pragma unroll
        for (int kk = 0; kk < KH; ++kk) acc = __builtin_fma((double)s_q[half * KH + kk], (double)wv[kk], acc);
        if (half) s_part[c] = acc;
        __syncthreads();
        if (!half) s_out[c] = (float)(acc + s_part[c]);
    }
    __syncthreads();
    if (tid < 64) { // both half-waves of wave 0 take the row; the first stores it
        const int l32 = tid & 31;
        float x[1][4];
#pragma unroll
        for (int t = 0; t < 4; ++t) x[0][t] = s_out[4 * l32 + t];
        int e[1];
        uint32_t cw[1];
        rotate_quantize<1>(x, l32, e, cw);
        if (tid < 32) {
            *(uint32_t *)(codes + m * R + c0 + 4 * l32) = cw[0];
            if (l32 == 0) qscales[m * NSEG + g] = exp2i(e[0]);
        }
    }
}

// ---------------------------------------------------------------------------
// Decode scoring from the FP8 cache.  Workgroup = 4 waves of one query; wave
// w streams tiles row0 + (w + 4 i) * 32 through a private ring of NB slots,
// each the tile's codes (32 rows x R bytes, 16-byte pieces XOR-swizzled by
// row) plus its rows' segment scales.  The query's codes are MFMA A
// fragments for the whole stream; the tile is the B operand; both scales
// enter as E8M0 exponents of v_mfma_scale_f32_32x32x64_f8f6f4.  With one
// wave per SIMD, the vector work of a tile delays the next DMA issue: over
// contiguous prefixes the DMA takes a scalar base plus fixed lane offsets,
// and the tile loop is unrolled over the ring so that every LDS address is
// a fixed lane offset plus an immediate.
// ---------------------------------------------------------------------------
typedef int i32x8 __attribute__((ext_vector_type(8)));

// The query of an FP8 decode launch into LDS, once per workgroup: wave w
// moves the codes of heads 16w .. 16w+15 (rows past H repeat row H-1 and are
// zeroed when read) into the last slot of its ring, which the stream does not
// touch before its (NB-1)-th tile, the 16-byte pieces of head h's row
// rotated by h so that the A-fragment reads (32 heads, the same piece) fall
// in distinct banks; wave 0 also moves the segment scales, wave 1 the head
// weights, wave 2 the heads' decoder biases (when there are any).  Returns
// the number of loads this wave issued.
template <int R, int HB, int NB, int SLOT>
__device__ __forceinline__ int stage_query_fp8(const uint8_t *qc, const float *qs, const float *wq, const float *bq,
                                               int H, lds_u8 *ring, lds_u8 *s_qs, lds_u8 *s_w, lds_u8 *s_b)
{
    constexpr int PR = R / 16;         // 16-byte pieces per row of codes
    constexpr int NIC = 16 * R / 1024; // 16 rows, 1 KiB per instruction
    constexpr int NSEG = R / kSeg;
    static_assert(SLOT >= 16 * R, "a ring slot holds 16 rows of query codes");
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int issued = 0;
    if (wv * 16 < HB * 32) {
        lds_u8 *slot = ring + (wv * NB + NB - 1) * SLOT;
#pragma unroll
        for (int ii = 0; ii < NIC; ++ii) {
            const int p = ii * 64 + lane;
            const int h = wv * 16 + p / PR, cs = p % PR;
            const int hs = h < H ? h : H - 1;
            dma16(qc + (int64_t)hs * R + (cs ^ (h & (PR - 1))) * 16, slot + ii * 1024);
        }
        issued = NIC;
    }
    if (wv == 0) {
#pragma unroll
        for (int g = 0; g < NSEG; ++g) {
            const int e = g * 64 + lane;
            dma4(qs + (e < H * NSEG ? e : H * NSEG - 1), s_qs + g * 256);
        }
        issued += NSEG;
    }
    if (wv == 1) {
        dma4(wq + (lane < H ? lane : H - 1), s_w);
        ++issued;
    }
    if (wv == 2 && bq) {
        dma4(bq + (lane < H ? lane : H - 1), s_b);
        ++issued;
    }
    return issued;
}

// The staged query into registers (after the workgroup barrier that follows
// its staging): A fragments, segment scales as E8M0 exponents, weights and
// biases, heads past H zero (their scales 2^0).
template <int R, int HB, int NB, int SLOT>
__device__ __forceinline__ void read_query_fp8(const lds_u8 *ring, const lds_f32 *s_qs, const lds_f32 *s_w,
                                               const lds_f32 *s_b, bool has_bias, int H, i32x8 (&qa)[HB][R / 64],
                                               int (&sa)[HB][R / kSeg], float (&wr)[HB][16], f32x16 (&br)[HB])
{
    constexpr int PR = R / 16;
    constexpr int KS = R / 64;
    constexpr int NSEG = R / kSeg;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        const int h = hb * 32 + (lane & 31);
        const bool live = h < H;
        const lds_u8 *row = ring + ((h >> 4) * NB + NB - 1) * SLOT + (h & 15) * R;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int p0 = 4 * s + 2 * (lane >> 5);
            const u32x4 lo = *(const lds_u32x4 *)(row + (p0 ^ (h & (PR - 1))) * 16);
            const u32x4 hi = *(const lds_u32x4 *)(row + ((p0 + 1) ^ (h & (PR - 1))) * 16);
            i32x8 v = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            if (!live) {
                i32x8 z = {};
                v = z;
            }
            qa[hb][s] = v;
        }
#pragma unroll
        for (int g = 0; g < NSEG; ++g) {
            const uint32_t e = (__float_as_uint(s_qs[(live ? h : 0) * NSEG + g]) >> 23) & 0xFFu;
            sa[hb][g] = live ? (int)e : 127;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int hh = hb * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            wr[hb][r] = hh < H ? s_w[hh] : 0.0f;
            br[hb][r] = has_bias && hh < H ? s_b[hh] : 0.0f;
        }
    }
}

template <int R, int HB, bool GATHER, int NB, bool NT>
__global__ __launch_bounds__(256) void k_score_fp8(ScoreArgs a, const float *pool_scales, int64_t qscale_off,
                                                   int tiles_per_wave)
{
    constexpr int NSEG = R / kSeg;
    constexpr int CODE_BYTES = kTile * R;      // one tile's codes
    constexpr int SLOT = CODE_BYTES + 256;     // + 32 rows x NSEG scales
    constexpr int NIC = CODE_BYTES / 1024;     // 1-KiB DMA instructions per tile
    constexpr int NIT = NIC + 1;               // + the scales
    constexpr int CH = R / 16;                 // 16-byte pieces per row
    constexpr int KS = R / 64;                 // MFMA k-steps
    constexpr int MAXT = GATHER ? kGatherTilesF8 : kMaxTilesPerWaveF8; // tiles per wave (scores kept in LDS)
    static_assert(4 * NB * SLOT + (GATHER ? 4 * kGatherTilesF8 * kTile * 4 : 0) + kHistBins * 4 +
                          4 * MAXT * kTile * 4 <= 160 * 1024,
                  "LDS budget");
    __shared__ __attribute__((aligned(1024))) uint8_t ring_raw[4 * NB * SLOT];
    __shared__ int32_t s_row[GATHER ? 4 * kGatherTilesF8 * kTile : 1];
    __shared__ uint32_t s_hist[kHistBins];
    __shared__ float s_out[4 * MAXT * kTile];
    // contiguous mode: the guessed sequence's page ids (wave w, lane i: its
    // tile i) and the query's scales, weights and biases, staged by DMA
    __shared__ int32_t s_pg[GATHER ? 1 : 4 * 64];
    __shared__ float s_qs[GATHER ? 1 : 64 * NSEG];
    __shared__ float s_w[GATHER ? 1 : 64];
    __shared__ float s_b[GATHER ? 1 : 64];

    const int q = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    LI_PHASE_DECL;
    LI_PHASE_START;
    // The query: codes as A fragments (lane l: head l%32 of block hb, k-block
    // l/32 of each 64-code step), segment scales as E8M0 exponents, weights.
    // Gather mode loads them per lane, first, beside the sequence id and the
    // candidates, and waits for them with those before any tile is issued:
    // one round trip for all of the start-up loads (waiting for per-lane
    // loads once tiles are in flight would also wait for every tile issued
    // before them).  Contiguous mode stages them through LDS by DMA instead
    // (below), so that the first tiles go out as soon as the page ids are in.
    i32x8 qa[HB][KS];
    int sa[HB][NSEG];
    float wr[HB][16];
    f32x16 br[HB]; // accumulator start values: each head's decoder bias (0 without one)
    const uint8_t *qc = (const uint8_t *)a.qt + (int64_t)q * a.H * R;
    const float *qs = (const float *)((const uint8_t *)a.qt + qscale_off) + (int64_t)q * a.H * NSEG;
    if constexpr (GATHER) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            const int h = hb * 32 + (lane & 31);
            const int hc = h < a.H ? h : a.H - 1;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const uint8_t *p = qc + (int64_t)hc * R + s * 64 + (lane >> 5) * 32;
                const u32x4 lo = *(const u32x4 *)p, hi = *(const u32x4 *)(p + 16);
                i32x8 v = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                if (h >= a.H) {
                    i32x8 z = {};
                    v = z;
                }
                qa[hb][s] = v;
            }
            // every load is unconditional (indices clamped into the query),
            // so they are all in flight together; heads past H are zeroed after
#pragma unroll
            for (int g = 0; g < NSEG; ++g) {
                const uint32_t e = (__float_as_uint(qs[(int64_t)hc * NSEG + g]) >> 23) & 0xFFu;
                sa[hb][g] = h < a.H ? (int)e : 127;
            }
            const float *wq = a.w + (int64_t)q * a.H;
            const float *bq = a.bias ? a.bias + (int64_t)q * a.H : a.w + (int64_t)q * a.H;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int hh = hb * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                const int hcl = hh < a.H ? hh : a.H - 1;
                const float wv_ = wq[hcl], bv_ = bq[hcl];
                wr[hb][r] = hh < a.H ? wv_ : 0.0f;
                br[hb][r] = a.bias && hh < a.H ? bv_ : 0.0f;
            }
        }
    }
    const int64_t row0 = (int64_t)blockIdx.x * 4 * tiles_per_wave * kTile;
    const int64_t first = row0 + (int64_t)wv * kTile;
    auto tile_row0 = [&](int i) -> int64_t { return first + (int64_t)i * 4 * kTile; };
    const int nt_max =
        first < a.max_rows ? (int)min64(tiles_per_wave, (a.max_rows - first + 4 * kTile - 1) / (4 * kTile)) : 0;

    // Contiguous mode: lane i holds the page id of this wave's tile i (at
    // most 64 tiles per wave); query q usually sits in sequence q, so that
    // block-table row is requested first, by LDS DMA, before the sequence id
    // arrives and ahead of the query staging.
    const int b_guess = q < a.batch ? q : 0;
    int staged = 0;
    if constexpr (!GATHER) {
        const int pidx = (int)min64(tile_row0(lane < nt_max ? lane : 0) >> 6, a.max_pages - 1);
        dma4(a.bt + (int64_t)b_guess * a.max_pages + pidx, (lds_u8 *)(s_pg + wv * 64));
        staged = stage_query_fp8<R, HB, NB, SLOT>(qc, qs, a.w + (int64_t)q * a.H,
                                                  a.bias ? a.bias + (int64_t)q * a.H : nullptr, a.H,
                                                  (lds_u8 *)ring_raw, (lds_u8 *)s_qs, (lds_u8 *)s_w, (lds_u8 *)s_b);
    }
    const int b = clamp_index(((const_i32_t *)a.qseq)[q], a.batch);
    int n = GATHER ? min(((const_i32_t *)a.cand_count)[q], (int)a.cand_ld)
                   : valid_rows(((const_i32_t *)a.qpos)[q], ((const_i32_t *)a.seq_lens)[b]);
    n = (int)min64(n, a.max_rows);
    const uint8_t *pool = (const uint8_t *)a.pool;
    lds_u8 *const ring = (lds_u8 *)ring_raw + wv * NB * SLOT;
    auto clamp_page = [&](int page) { return page < 0 ? 0 : (page < a.num_pages ? page : a.num_pages - 1); };
    int tile_page = 0;
    if constexpr (!GATHER) {
        wait_vmcnt_upto(staged); // the page ids have landed (vector loads complete in issue order)
        if (b == b_guess)
            tile_page = ((const __attribute__((address_space(3))) int32_t *)s_pg)[wv * 64 + lane];
        else if (lane < nt_max)
            tile_page = a.bt[(int64_t)b * a.max_pages + (tile_row0(lane) >> 6)];
        tile_page = clamp_page(tile_page);
    }

    if constexpr (GATHER) {
        // physical slots of every tile row of this wave, two batched rounds
        const int64_t max_pos = (int64_t)a.max_pages * kPage - 1;
        int pos[kGatherTilesF8], page[kGatherTilesF8];
#pragma unroll
        for (int i = 0; i < kGatherTilesF8; ++i) {
            pos[i] = 0;
            if (i < nt_max) {
                int64_t j = tile_row0(i) + (lane & 31);
                j = j < a.cand_ld ? j : a.cand_ld - 1;
                pos[i] = a.cand[(int64_t)q * a.cand_ld + j];
            }
        }
#pragma unroll
        for (int i = 0; i < kGatherTilesF8; ++i) {
            pos[i] = pos[i] < 0 ? 0 : (pos[i] > max_pos ? (int)max_pos : pos[i]);
            page[i] = 0;
            if (i < nt_max) page[i] = a.bt[(int64_t)b * a.max_pages + (pos[i] >> 6)];
        }
#pragma unroll
        for (int i = 0; i < kGatherTilesF8; ++i)
            if (i < nt_max && lane < 32)
                s_row[(wv * kGatherTilesF8 + i) * kTile + lane] = clamp_page(page[i]) * kPage + (pos[i] & 63);
        wait_lds();
    }
    uint32_t src_off[NIC];
#pragma unroll
    for (int ii = 0; ii < NIC; ++ii) {
        const int p = ii * 64 + lane;
        const int nr = p / CH, cs = p % CH;
        src_off[ii] = (uint32_t)(nr * R + (cs ^ (nr % CH)) * 16);
    }
    uint32_t sc_src_off;
    {
        int sl = lane / NSEG;
        sl = sl < kTile ? sl : kTile - 1;
        sc_src_off = (uint32_t)((sl * NSEG + lane % NSEG) * 4);
    }
    // tile i -> slot (i % NB): the codes, then the scales of its 32 rows
    auto issue = [&](int i, int slot_idx) {
        lds_u8 *slot = ring + slot_idx * SLOT;
        const __attribute__((address_space(3))) int32_t *rows =
            (const __attribute__((address_space(3))) int32_t *)s_row + (wv * kGatherTilesF8 + i) * kTile;
        int64_t base = 0;
        if constexpr (!GATHER) {
            const int64_t t0 = tile_row0(i);
            base = (int64_t)__builtin_amdgcn_readlane(tile_page, i) * kPage + (t0 & 63);
        }
        auto slot_of = [&](int nr) -> int64_t {
            if constexpr (GATHER) return (int64_t)rows[nr];
            else return base + nr;
        };
        if constexpr (GATHER) {
#pragma unroll
            for (int ii = 0; ii < NIC; ++ii) {
                const int p = ii * 64 + lane;
                const int nr = p / CH, cs = p % CH;
                const int c = cs ^ (nr % CH);
                dma16p<NT>(pool + slot_of(nr) * R + c * 16, slot + ii * 1024);
            }
            int sl = lane / NSEG;
            sl = sl < kTile ? sl : kTile - 1;
            dma4(pool_scales + slot_of(sl) * NSEG + (lane % NSEG), slot + CODE_BYTES);
        } else {
            const uint8_t *gcode = pool + base * R;
            const uint8_t *gscale = (const uint8_t *)(pool_scales + base * NSEG);
#pragma unroll
            for (int ii = 0; ii < NIC; ++ii) dma16s<NT>(gcode, src_off[ii], slot + ii * 1024);
            dma4s(gscale, sc_src_off, slot + CODE_BYTES);
        }
    };
    const int npro = min(NB - 1, nt_max);
    if constexpr (GATHER) {
        // every start-up load (query, weights, gathered rows) has landed:
        // s_waitcnt vmcnt(0), issued as the builtin so that the compiler
        // counts it and adds no wait of its own for these loads later
        __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    for (int i = 0; i < npro; ++i) issue(i, i);
    if constexpr (!GATHER) {
        // the query staging was issued before these tiles, so it has landed
        // once at most they are outstanding; every wave's part, then the
        // registers, then no wave reuses a staging slot before all have read
        wait_after<NIT, NB - 1>(npro);
        wg_barrier();
        read_query_fp8<R, HB, NB, SLOT>((const lds_u8 *)ring_raw, (const lds_f32 *)s_qs, (const lds_f32 *)s_w,
                                        (const lds_f32 *)s_b, a.bias != nullptr, a.H, qa, sa, wr, br);
        wait_lds();
        wg_barrier();
    }

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
    if (a.hist) wg_barrier(); // histogram cleared before any wave counts into it

    __attribute__((address_space(3))) float *const outw =
        (__attribute__((address_space(3))) float *)s_out + wv * kTile;
    const int nr = lane & 31, gk = lane >> 5;
    uint32_t rd_off[KS][2];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int c = 4 * s + 2 * gk;
        rd_off[s][0] = (uint32_t)((nr * CH + (c ^ (nr % CH))) * 16);
        rd_off[s][1] = (uint32_t)((nr * CH + ((c + 1) ^ (nr % CH))) * 16);
    }
    // The head sum of a tile runs one tile late: tile i's MFMAs issue first
    // and tile i-1's ReLU-weighted sum (registers only) follows while they
    // execute.  Tile i accumulates into accs[i & 1]; the loop is unrolled
    // over lcm(NB, 2) tiles so that both the ring slot and the set are
    // compile-time constants.  Both lane halves end with the row's whole
    // score, so lane l and lane l + 32 store the same value to the same LDS
    // word and the store needs no branch (rows past n are never read back).
    f32x16 accs[2][HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) accs[0][hb] = accs[1][hb] = f32x16{};
    auto tile = [&](auto Uc, int i) {
        constexpr int U = decltype(Uc)::value;
        constexpr int SL = U % NB;
        constexpr int NX = (SL + NB - 1) % NB;
        constexpr int PAR = U & 1;
        if (i + NB - 1 < nt) {
            wait_lds(); // this wave's reads of that slot (tile i-1) are complete
            issue(i + NB - 1, NX);
        }
        wait_after<NIT, NB - 1>(min(NB - 1, nt - 1 - i));
        LI_PHASE_FIRST_IF(i == 0);
        const lds_u8 *slot = ring + SL * SLOT;
        int sb[NSEG];
#pragma unroll
        for (int g = 0; g < NSEG; ++g)
            sb[g] = (int)((*(const __attribute__((address_space(3))) uint32_t *)(slot + CODE_BYTES +
                                                                                  (nr * NSEG + g) * 4) >> 23) & 0xFFu);
        f32x16(&acc)[HB] = accs[PAR];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const u32x4 lo = *(const lds_u32x4 *)(slot + rd_off[s][0]);
            const u32x4 hi = *(const lds_u32x4 *)(slot + rd_off[s][1]);
            const i32x8 bv = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            const int g = (s * 64) / kSeg;
#pragma unroll
            for (int hb = 0; hb < HB; ++hb)
                acc[hb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[hb][s], bv, s == 0 ? br[hb] : acc[hb], 0, 0,
                                                                          0, sa[hb][g], 0, sb[g]);
        }
        // tile i-1's sum, interleaved with the MFMAs above (for i = 0 a sum
        // over zeroed accumulators, written to tile 0's words, which tile 0's
        // own score overwrites one tile later)
        const float p = epilogue<HB>(accs[PAR ^ 1], wr);
        __builtin_amdgcn_sched_group_barrier(0x100, KS * 2 + 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, NSEG, 0);
        static_for<KS * HB>([&](auto) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 40 / KS, 0);
        });
        outw[(i > 0 ? i - 1 : 0) * 4 * kTile + (lane & 31)] = p; // local row ((i-1) * 4 + wv) * 32 + lane
    };
    constexpr int UN = NB % 2 == 0 ? NB : 2 * NB;
#pragma unroll 1
    for (int i0 = 0; i0 < nt; i0 += UN)
        static_for<UN>([&](auto Uc) {
            const int i = i0 + decltype(Uc)::value;
            if (i < nt) tile(Uc, i);
        });
    if (nt > 0) {
        const float p = (nt - 1) & 1 ? epilogue<HB>(accs[1], wr) : epilogue<HB>(accs[0], wr);
        outw[(nt - 1) * 4 * kTile + (lane & 31)] = p;
    }
    wait_vmcnt<0>(); // tiles issued ahead of the row count and never used
    LI_PHASE_LOOP;
    __syncthreads(); // every wave's scores are in LDS (and the histogram is cleared)
    LI_PHASE_SYNC;
    // The scores leave in one coalesced pass over the workgroup's rows (score
    // stores among the stream's loads interleave DRAM writes with the read
    // stream), which also counts their first radix digit; the fused filter
    // pass follows when asked for.
    const int rows = (int)min64(4 * (int64_t)tiles_per_wave * kTile, n - row0);
    score_tail(a, q, row0, rows, n, (const lds_f32 *)s_out, s_hist, (FilterLds *)ring_raw);
    LI_PHASE_STORE(g_phase_fp8, wv, lane);
}

// ---------------------------------------------------------------------------
// Prefill scoring from the FP8 cache: workgroup = 4 consecutive queries (one
// per wave) sharing every tile through an NBUF-deep LDS ring, one barrier
// per tile, page ids staged in LDS per split; the same slot layout and
// scaled MFMA as the decode kernel.  Each wave moves a quarter of a tile's
// codes and a quarter of its scales.  No first-digit counting here (the
// selection pass counts it), so two workgroups share a CU.
// ---------------------------------------------------------------------------
constexpr int kPrefillMaxTilesF8 = 2048; // max tiles per split (their page ids sit in LDS)

template <int R, int HB, int NBUF, bool BIAS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_score_prefill_fp8(
    ScoreArgs a, const float *pool_scales, int64_t qscale_off, int tiles_per_split)
{
    constexpr int NSEG = R / kSeg;
    constexpr int CODE_BYTES = kTile * R;
    constexpr int SLOT = CODE_BYTES + 256;
    constexpr int NIC = CODE_BYTES / 1024;
    constexpr int NIW = NIC / 4;           // code DMA instructions per wave per tile
    constexpr int CH = R / 16;
    constexpr int KS = R / 64;
    static_assert(NIW >= 1, "tile must split over 4 waves");
    static_assert(NBUF % 2 == 0, "a tile's accumulator set is its ring slot's parity");
    __shared__ __attribute__((aligned(1024))) uint8_t ring_raw[NBUF * SLOT];
    __shared__ int32_t s_page_raw[kPrefillMaxTilesF8 / 2 + 2];
    lds_u8 *ring = (lds_u8 *)ring_raw;
    lds_i32 *s_page = (lds_i32 *)s_page_raw;

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
        sb[u] = qq < a.Q ? clamp_index(qseq[qq], a.batch) : -1;
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
    // this wave's query (zero codes past the batch)
    i32x8 qa[HB][KS];
    int sa[HB][NSEG];
    float wr[HB][16];
    f32x16 br[HB]; // accumulator start values: each head's decoder bias (0 without one)
    {
        const bool live = q < a.Q;
        const int qc_i = live ? q : 0;
        const uint8_t *qc = (const uint8_t *)a.qt + (int64_t)qc_i * a.H * R;
        const float *qs = (const float *)((const uint8_t *)a.qt + qscale_off) + (int64_t)qc_i * a.H * NSEG;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            const int h = hb * 32 + (lane & 31);
            const bool hv = live && h < a.H;
            const int hc = h < a.H ? h : a.H - 1;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const uint8_t *p = qc + (int64_t)hc * R + s * 64 + (lane >> 5) * 32;
                const u32x4 lo = *(const u32x4 *)p, hi = *(const u32x4 *)(p + 16);
                i32x8 v = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                if (!hv) {
                    i32x8 z = {};
                    v = z;
                }
                qa[hb][s] = v;
            }
#pragma unroll
            for (int g = 0; g < NSEG; ++g)
                sa[hb][g] = hv ? (int)((__float_as_uint(qs[(int64_t)hc * NSEG + g]) >> 23) & 0xFFu) : 127;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int hh = hb * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                wr[hb][r] = live && hh < a.H ? a.w[(int64_t)qc_i * a.H + hh] : 0.0f;
                br[hb][r] = live && a.bias && hh < a.H ? a.bias[(int64_t)qc_i * a.H + hh] : 0.0f;
            }
        }
    }
    float *out = a.out + (int64_t)(q < a.Q ? q : 0) * a.out_ld;
    // this query's scores as a raw buffer of my_n floats (bounds-checked)
    const __amdgpu_buffer_rsrc_t out_rsrc = __builtin_amdgcn_make_buffer_rsrc(out, 0, my_n * 4, kBufferWord3);
    const uint8_t *pool = (const uint8_t *)a.pool;
    const int nr = lane & 31, gk = lane >> 5;
    // Per-lane parts of every tile's addresses, the same for every tile:
    // byte offsets of this lane's DMA sources inside a tile's codes and
    // scales, and LDS offsets (inside a slot) of its MFMA B fragments (rows
    // swizzled across the 16-byte columns) and of its row's scales.
    uint32_t src_off[NIW];
#pragma unroll
    for (int j = 0; j < NIW; ++j) {
        const int p = (wv * NIW + j) * 64 + lane;
        const int rr = p / CH, cs = p % CH;
        src_off[j] = (uint32_t)(rr * R + (cs ^ (rr % CH)) * 16);
    }
    uint32_t sc_src_off;
    {
        const int f = wv * 16 + (lane & 15);
        const int row = f / NSEG < kTile ? f / NSEG : kTile - 1;
        sc_src_off = (uint32_t)((row * NSEG + f % NSEG) * 4);
    }
    uint32_t rd_off[KS][2];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int c = 4 * s + 2 * gk;
        rd_off[s][0] = (uint32_t)((nr * CH + (c ^ (nr % CH))) * 16);
        rd_off[s][1] = (uint32_t)((nr * CH + ((c + 1) ^ (nr % CH))) * 16);
    }
    uint32_t sc_rd_off[NSEG];
#pragma unroll
    for (int g = 0; g < NSEG; ++g) sc_rd_off[g] = (uint32_t)(CODE_BYTES + (nr * NSEG + g) * 4);

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
        const int p0 = ts >> 1;
        const int np = ((te - 1) >> 1) - p0 + 1;
        __syncthreads(); // the previous pass is done with the ring and the page ids
        for (int pi = threadIdx.x; pi < np; pi += 256)
            s_page[pi] = clamp_index(a.bt[(int64_t)b * a.max_pages + p0 + pi], a.num_pages);
        __syncthreads();
        // page ids are wave-uniform: read once into scalar registers
        auto page_of = [&](int i) { return __builtin_amdgcn_readfirstlane(s_page[((ts + i) >> 1) - p0]); };
        auto issue = [&](int i, int page, int slot_idx) {
            const int64_t base = (int64_t)page * kPage + ((ts + i) & 1) * kTile; // first row of the tile
            const uint8_t *gcode = pool + base * R;
            const uint8_t *gscale = (const uint8_t *)(pool_scales + base * NSEG);
            lds_u8 *slot = ring + slot_idx * SLOT;
#pragma unroll
            for (int j = 0; j < NIW; ++j) dma16s(gcode, src_off[j], slot + (wv * NIW + j) * 1024);
            // scales: this wave's quarter (16 lanes x 4 bytes) of the tile's 32 x NSEG
            if (lane < 16) dma4s(gscale, sc_src_off, slot + CODE_BYTES + wv * 64);
        };
        // The epilogue of a tile runs one tile late: the MFMAs of tile i
        // issue first and the ReLU-weighted head sum of tile i-1 (registers
        // only) follows while they execute, so the vector work overlaps the
        // matrix core instead of waiting for it.  Tile i accumulates into
        // accs[i & 1] (the ring depth is even, so that is the slot's parity).
        f32x16 accs[2][HB];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) accs[0][hb] = accs[1][hb] = f32x16{};
        auto finish = [&](const f32x16 (&acc)[HB], int i) {
            const float pv = epilogue<HB>(acc, wr);
            const int j = (ts + i) * kTile + lane;
            if (lane < 32 && j < my_n) out[j] = pv;
        };
        // One tile; its ring slot SL (and that of the tile issued in its
        // place) is a compile-time constant, so every LDS address below is a
        // fixed per-lane offset plus an immediate.
        auto tile = [&](auto SLc, int i) {
            constexpr int SL = decltype(SLc)::value;
            constexpr int NX = (SL + NBUF - 1) % NBUF; // slot of tile i + NBUF - 1 (tile i-1's)
            const int inext = i + NBUF - 1;
            const int pnext = inext < nt ? page_of(inext) : 0; // read before the barrier
            // tile i landed (this wave's part), tiles i+1..i+NBUF-2 may still fly
            wait_after<NIW + 1, NBUF - 2>(min(NBUF - 2, nt - 1 - i));
            wg_barrier(); // every part of tile i landed; every wave is done with tile i-1
            if (inext < nt) issue(inext, pnext, NX);
            if (active) {
                const lds_u8 *slot = ring + SL * SLOT;
                int scb[NSEG];
#pragma unroll
                for (int g = 0; g < NSEG; ++g)
                    scb[g] = (int)((*(const __attribute__((address_space(3))) uint32_t *)(slot + sc_rd_off[g]) >> 23) &
                                   0xFFu);
                // accumulators start from the heads' biases, or (no bias) the
                // first step adds to a constant zero
                f32x16(&acc)[HB] = accs[SL & 1];
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const u32x4 lo = *(const lds_u32x4 *)(slot + rd_off[s][0]);
                    const u32x4 hi = *(const lds_u32x4 *)(slot + rd_off[s][1]);
                    const i32x8 bv = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                      (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                    const int g = (s * 64) / kSeg;
#pragma unroll
                    for (int hb = 0; hb < HB; ++hb) {
                        const f32x16 zero = {};
                        acc[hb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            qa[hb][s], bv, s == 0 ? (BIAS ? br[hb] : zero) : acc[hb], 0, 0, 0, sa[hb][g], 0, scb[g]);
                    }
                }
                // tile i-1's head sum (for i = 0 a discarded sum of zeros)
                const float pv = epilogue<HB>(accs[(SL + 1) & 1], wr);
                // issue order: the fragment reads, then each MFMA followed by
                // a share of the head sum's vector instructions
                __builtin_amdgcn_sched_group_barrier(0x100, KS * 2 + 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, NSEG, 0);
                static_for<KS * HB>([&](auto) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 40 / KS, 0);
                });
                // a buffer store whose out-of-range offsets the hardware
                // drops: no branch, so the MFMAs and the sum stay together
                const int j = (ts + i - 1) * kTile + lane;
                const bool ok = i > 0 && lane < 32 && j < my_n;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pv), out_rsrc, ok ? j * 4 : kBufferDrop, 0, 0);
            }
        };
        for (int i = 0; i < NBUF - 1 && i < nt; ++i) issue(i, page_of(i), i);
#pragma unroll 1
        for (int i0 = 0; i0 < nt; i0 += NBUF)
            static_for<NBUF>([&](auto SLc) {
                const int i = i0 + decltype(SLc)::value;
                if (i < nt) tile(SLc, i);
            });
        if (active) {
            if ((nt - 1) & 1)
                finish(accs[1], nt - 1);
            else
                finish(accs[0], nt - 1);
        }
    }
}

template <int R, int HB>
hipError_t launch_prefill_fp8_rh(const ScoreArgs &a, const float *pool_scales, int64_t qscale_off, int64_t max_rows,
                                 hipStream_t s)
{
    constexpr int NBUF = 6;
    const int64_t tiles = (max_rows + kTile - 1) / kTile;
    const int qblocks = (a.Q + 3) / 4;
    int64_t splits = 1;
    if (qblocks < 512) splits = std::min<int64_t>((512 + qblocks - 1) / qblocks, tiles);
    if (splits < 1) splits = 1;
    int64_t tps = (tiles + splits - 1) / splits;
    if (tps > kPrefillMaxTilesF8) tps = kPrefillMaxTilesF8;
    splits = (tiles + tps - 1) / tps;
    const dim3 grid(qblocks, (unsigned)splits);
    if (a.bias)
        return launch_kernel(k_score_prefill_fp8<R, HB, NBUF, true>, grid, dim3(256), 0, s, a, pool_scales, qscale_off,
                             (int)tps);
    return launch_kernel(k_score_prefill_fp8<R, HB, NBUF, false>, grid, dim3(256), 0, s, a, pool_scales, qscale_off,
                         (int)tps);
}

template <int R, int HB>
hipError_t launch_score_fp8_rh(const ScoreArgs &a, const float *pool_scales, int64_t qscale_off, int64_t max_rows,
                               hipStream_t s, bool *filtered)
{
    // ring next to the histogram, the staged scores (64 tiles per wave, 16 in
    // gather mode) and, in gather mode, the row table: 3 slots at r = 256,
    // 6 at r = 128 (7 in gather mode).  Measured: a 4-slot ring with 16 tiles
    // per wave was no faster at 4 x 131072 rows and 19% slower at 16 x 131072
    // (four times the workgroups).
    constexpr int NB = R == 256 ? 3 : 6;
    constexpr int NBG = R == 256 ? 3 : 7;
    const int64_t tiles = (max_rows + kTile - 1) / kTile;
    const int64_t per_q = (256 + a.Q - 1) / a.Q;
    int64_t tpw = (tiles + 4 * per_q - 1) / (4 * per_q);
    if (tpw < 1) tpw = 1;
    if (a.cand && tpw > kGatherTilesF8) tpw = kGatherTilesF8;
    if (!a.cand && tpw > kMaxTilesPerWaveF8) tpw = kMaxTilesPerWaveF8;
    const int64_t wgs = (tiles + 4 * tpw - 1) / (4 * tpw);
    const dim3 grid((unsigned)wgs, a.Q);
    // the filter pass rides along when every workgroup of the grid is resident
    ScoreArgs b = a;
    b.flt.on = a.flt.on && !a.cand && a.hist && fused_filter_fits(wgs, a.Q);
    if (filtered) *filtered = b.flt.on;
    if (b.cand)
        return launch_kernel(k_score_fp8<R, HB, true, NBG, false>, grid, dim3(256), 0, s, b, pool_scales, qscale_off,
                             (int)tpw);
    if (b.stream_nt)
        return launch_kernel(k_score_fp8<R, HB, false, NB, true>, grid, dim3(256), 0, s, b, pool_scales, qscale_off,
                             (int)tpw);
    return launch_kernel(k_score_fp8<R, HB, false, NB, false>, grid, dim3(256), 0, s, b, pool_scales, qscale_off,
                         (int)tpw);
}

template <int R>
hipError_t launch_score_fp8_r(const ScoreArgs &a, const float *pool_scales, int64_t qscale_off, bool prefill,
                              int64_t max_rows, hipStream_t s, bool *filtered)
{
    if (prefill) {
        if (a.H <= 32) return launch_prefill_fp8_rh<R, 1>(a, pool_scales, qscale_off, max_rows, s);
        return launch_prefill_fp8_rh<R, 2>(a, pool_scales, qscale_off, max_rows, s);
    }
    if (a.H <= 32) return launch_score_fp8_rh<R, 1>(a, pool_scales, qscale_off, max_rows, s, filtered);
    return launch_score_fp8_rh<R, 2>(a, pool_scales, qscale_off, max_rows, s, filtered);
}

template <int R, int D, bool IDENT = false>
void launch_absorb_fp8_rd(const u16 *q, const u16 *W, uint8_t *codes, float *scales, int64_t QH, hipStream_t s)
{
    // many rows: big register tiles; few rows: small blocks, more workgroups;
    // decode-sized: a workgroup per row segment
    if (QH <= kAbsorbRowMax) {
        hipLaunchKernelGGL((k_absorb_fp8_row<R, D, IDENT>), dim3((unsigned)QH, R / kSeg), dim3(256), 0, s, q, W, codes,
                           scales);
        return;
    }
    if ((QH + 127) / 128 >= 256)
        hipLaunchKernelGGL((k_absorb_fp8<R, D, 128, IDENT>), dim3((unsigned)((QH + 127) / 128), R / kSeg), dim3(256),
                           0, s, q, W, codes, scales, QH);
    else if ((QH + 31) / 32 >= 64)
        hipLaunchKernelGGL((k_absorb_fp8<R, D, 32, IDENT>), dim3((unsigned)((QH + 31) / 32), R / kSeg), dim3(256), 0,
                           s, q, W, codes, scales, QH);
    else
        hipLaunchKernelGGL((k_absorb_fp8<R, D, 8, IDENT>), dim3((unsigned)((QH + 7) / 8), R / kSeg), dim3(256), 0, s,
                           q, W, codes, scales, QH);
}

template <int R>
hipError_t launch_absorb_fp8_r(const u16 *q, const u16 *W, uint8_t *codes, float *scales, int64_t QH, int d,
                               hipStream_t s)
{
    switch (d) {
    case 32: launch_absorb_fp8_rd<R, 32>(q, W, codes, scales, QH, s); break;
    case 64: launch_absorb_fp8_rd<R, 64>(q, W, codes, scales, QH, s); break;
    case 128: launch_absorb_fp8_rd<R, 128>(q, W, codes, scales, QH, s); break;
    case 256: launch_absorb_fp8_rd<R, 256>(q, W, codes, scales, QH, s); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace

#ifdef LI_PHASE_PROBE
hipError_t phase_records_fp8(void **dev) { return hipGetSymbolAddress(dev, HIP_SYMBOL(g_phase_fp8)); }
#else
hipError_t phase_records_fp8(void **dev)
{
    *dev = nullptr;
    return hipErrorNotSupported;
}
#endif

int64_t fp8_query_scale_offset(int64_t Q, int64_t H, int64_t r) { return (Q * H * r + 255) / 256 * 256; }

hipError_t launch_append_fp8(void *pool, float *scales, const int32_t *bt, const PoolGeom &geo, int r, const void *rows,
                             const int32_t *seq, const int32_t *pos, int T, const RopeArgs &rope, hipStream_t s)
{
    if (T <= 0) return hipSuccess;
    const int64_t halves = (int64_t)T * (r / kSeg);
    const unsigned blocks = (unsigned)((halves * 32 + 255) / 256);
    if (r == 256)
        hipLaunchKernelGGL((k_append_fp8<256>), dim3(blocks), dim3(256), 0, s, (uint8_t *)pool, scales, bt, geo,
                           (const u16 *)rows, seq, pos, T, rope);
    else if (r == 128)
        hipLaunchKernelGGL((k_append_fp8<128>), dim3(blocks), dim3(256), 0, s, (uint8_t *)pool, scales, bt, geo,
                           (const u16 *)rows, seq, pos, T, rope);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_absorb_fp8(const void *q, const void *W, void *qt, int64_t QH, int d, int r, hipStream_t s)
{
    if (QH <= 0) return hipSuccess;
    uint8_t *codes = (uint8_t *)qt;
    float *scales = (float *)((uint8_t *)qt + fp8_query_scale_offset(QH, 1, r));
    const u16 *qq = (const u16 *)q, *ww = (const u16 *)W;
    if (!W) { // no decoder: the query (d == r) is rotated and quantized as it is
        if (d != r) return hipErrorInvalidValue;
        if (r == 256) launch_absorb_fp8_rd<256, 256, true>(qq, nullptr, codes, scales, QH, s);
        else if (r == 128) launch_absorb_fp8_rd<128, 128, true>(qq, nullptr, codes, scales, QH, s);
        else return hipErrorInvalidValue;
        return hipGetLastError();
    }
    if (r == 256) return launch_absorb_fp8_r<256>(qq, ww, codes, scales, QH, d, s);
    if (r == 128) return launch_absorb_fp8_r<128>(qq, ww, codes, scales, QH, d, s);
    return hipErrorInvalidValue;
}

hipError_t launch_score_fp8(const ScoreArgs &a, const float *pool_scales, int64_t qscale_off, int r,
                            bool many_queries_per_seq, int64_t max_rows, hipStream_t s, bool *filtered)
{
    if (filtered) *filtered = false;
    if (a.Q <= 0 || max_rows <= 0) return hipSuccess;
    const bool prefill = many_queries_per_seq && a.cand == nullptr && a.hist == nullptr;
    if (r == 256) return launch_score_fp8_r<256>(a, pool_scales, qscale_off, prefill, max_rows, s, filtered);
    if (r == 128) return launch_score_fp8_r<128>(a, pool_scales, qscale_off, prefill, max_rows, s, filtered);
    return hipErrorInvalidValue;
}

} // namespace li

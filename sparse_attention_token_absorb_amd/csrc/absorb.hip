// Query-side decoder absorption (gfx950).
//
// LatentIndex (paperlayer.ai summary of arXiv:2610.04635), §3.1, §A.2, §B.2:
// each layer folds its key decoder W_dec [d][r] into its query so that it
// scores the shared latent directly: qt[m][t] = sum_e q[m][e] W_dec[e][t]
// for every (query, head) row m.  A GEMM with M = queries*heads, K = d,
// N = r; bf16 inputs on v_mfma_f32_32x32x16_bf16 with fp32 accumulation and a
// single round-to-nearest-even to bf16 at the end.
//
// Both MFMA operands want K-contiguous fragments; q rows already are, W_dec is
// not, so every workgroup stages its column slice of W_dec transposed in LDS
// (row stride d + 8 halves keeps the fragment reads conflict-free) and reuses
// it for 128 rows.
#include "li_internal.hpp"

namespace li {
namespace {

template <int R, int D, int NC>
__global__ __launch_bounds__(256) void k_absorb_bf16(const u16 *q, const u16 *W, u16 *qt, int64_t QH)
{
    constexpr int LD = D + 8; // halves per transposed row
    constexpr int KS = D / 16;
    constexpr int ITEMS = (D / 2) * (NC / 8); // (row pair, 8 columns) pieces of this column slice of W
    constexpr int NIT = (ITEMS + 255) / 256;
    __shared__ __attribute__((aligned(16))) u16 wt[NC * LD];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int c0 = blockIdx.y * NC; // first column of W (and of qt) this workgroup covers
    const int64_t m0 = (int64_t)blockIdx.x * 128 + wv * 32;

    // A fragments (rows of q are K-contiguous already), issued first so their
    // latency overlaps the W loads.
    bf16x8 a[KS];
    {
        const int64_t m = m0 + (lane & 31);
        const int64_t mc = m < QH ? m : QH - 1;
#pragma unroll
        for (int s = 0; s < KS; ++s) a[s] = *(const bf16x8 *)(q + mc * D + s * 16 + (lane >> 5) * 8);
        if (m >= QH) {
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                bf16x8 z = {};
                a[s] = z;
            }
        }
    }
    // W[:, c0:c0+NC] -> wt [NC][LD] (transposed), two source rows per piece so
    // the LDS writes are 32-bit; all loads are issued before any write.
    bf16x8 r0[NIT], r1[NIT];
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
        int it = tid + k * 256;
        it = it < ITEMS ? it : ITEMS - 1;
        const int e = (it / (NC / 8)) * 2;
        const int t0 = c0 + (it % (NC / 8)) * 8;
        r0[k] = *(const bf16x8 *)(W + (int64_t)e * R + t0);
        r1[k] = *(const bf16x8 *)(W + (int64_t)(e + 1) * R + t0);
    }
#pragma unroll
    for (int k = 0; k < NIT; ++k) {
        const int it = tid + k * 256;
        if (it < ITEMS) {
            const int e = (it / (NC / 8)) * 2;
            const int tl = (it % (NC / 8)) * 8;
            const u16 *h0 = (const u16 *)&r0[k];
            const u16 *h1 = (const u16 *)&r1[k];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                *(uint32_t *)(wt + (tl + i) * LD + e) = (uint32_t)h0[i] | ((uint32_t)h1[i] << 16);
        }
    }
    __syncthreads();
    if (m0 >= QH) return;
#pragma unroll 1
    for (int nt = 0; nt < NC / 32; ++nt) {
        f32x16 acc = {};
        const int n = nt * 32 + (lane & 31);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const bf16x8 b = *(const bf16x8 *)(wt + n * LD + s * 16 + (lane >> 5) * 8);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b, acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t m = m0 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            if (m < QH) qt[m * R + c0 + n] = f32_to_bf16_rne(acc[r]);
        }
    }
}

__global__ __launch_bounds__(256) void k_absorb_f32(const float *q, const float *W, float *qt, int64_t QH, int d,
                                                    int r)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= QH * r) return;
    const int64_t m = i / r;
    const int t = (int)(i % r);
    float acc = 0.0f;
    for (int e = 0; e < d; ++e) acc = fmaf(q[m * d + e], W[(int64_t)e * r + t], acc);
    qt[i] = acc;
}

template <int R, int D>
void launch_rd(const u16 *q, const u16 *W, u16 *qt, int64_t QH, hipStream_t s)
{
    const int64_t mblocks = (QH + 127) / 128;
    if (mblocks >= 256) {
        // many rows (prefill): each workgroup covers all columns, W staged once per 128 rows
        hipLaunchKernelGGL((k_absorb_bf16<R, D, R>), dim3((unsigned)mblocks, 1), dim3(256), 0, s, q, W, qt, QH);
    } else {
        // few rows (decode): one 32-column slice per workgroup, so the W loads
        // and the MFMA work spread over R/32 times more workgroups
        hipLaunchKernelGGL((k_absorb_bf16<R, D, 32>), dim3((unsigned)mblocks, R / 32), dim3(256), 0, s, q, W, qt,
                           QH);
    }
}

template <int R>
hipError_t launch_bf16_r(const void *q, const void *W, void *qt, int64_t QH, int d, hipStream_t s)
{
    const u16 *qq = (const u16 *)q;
    const u16 *ww = (const u16 *)W;
    u16 *oo = (u16 *)qt;
    switch (d) {
    case 32: launch_rd<R, 32>(qq, ww, oo, QH, s); break;
    case 64: launch_rd<R, 64>(qq, ww, oo, QH, s); break;
    case 128: launch_rd<R, 128>(qq, ww, oo, QH, s); break;
    case 256: launch_rd<R, 256>(qq, ww, oo, QH, s); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace

hipError_t launch_absorb(const void *q, const void *W, void *qt, int64_t QH, int d, int r, bool bf16, hipStream_t s)
{
    if (QH <= 0) return hipSuccess;
    if (!bf16) {
        const int64_t n = QH * r;
        hipLaunchKernelGGL(k_absorb_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const float *)q,
                           (const float *)W, (float *)qt, QH, d, r);
        return hipGetLastError();
    }
    switch (r) {
    case 64: return launch_bf16_r<64>(q, W, qt, QH, d, s);
    case 128: return launch_bf16_r<128>(q, W, qt, QH, d, s);
    case 256: return launch_bf16_r<256>(q, W, qt, QH, d, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace li

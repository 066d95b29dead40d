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
// not, so every workgroup stages W_dec transposed in LDS (row stride d + 8
// halves keeps the fragment reads conflict-free) and reuses it for 128 rows.
#include "li_internal.hpp"

namespace li {
namespace {

template <int R, int D>
__global__ __launch_bounds__(256) void k_absorb_bf16(const u16 *q, const u16 *W, u16 *qt, int64_t QH)
{
    constexpr int LD = D + 8; // halves per transposed row
    constexpr int KS = D / 16;
    __shared__ __attribute__((aligned(16))) u16 wt[R * LD];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    // W [D][R] -> wt [R][LD], two source rows per item so LDS writes are 32-bit.
    for (int it = tid; it < (D / 2) * (R / 8); it += 256) {
        const int e = (it / (R / 8)) * 2;
        const int t0 = (it % (R / 8)) * 8;
        const bf16x8 r0 = *(const bf16x8 *)(W + (int64_t)e * R + t0);
        const bf16x8 r1 = *(const bf16x8 *)(W + (int64_t)(e + 1) * R + t0);
        const u16 *h0 = (const u16 *)&r0;
        const u16 *h1 = (const u16 *)&r1;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *(uint32_t *)(wt + (t0 + i) * LD + e) = (uint32_t)h0[i] | ((uint32_t)h1[i] << 16);
    }
    __syncthreads();
    const int64_t m0 = (int64_t)blockIdx.x * 128 + wv * 32;
    if (m0 >= QH) return;
    bf16x8 a[KS];
    {
        const int64_t m = m0 + (lane & 31);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (m < QH) {
                a[s] = *(const bf16x8 *)(q + m * D + s * 16 + (lane >> 5) * 8);
            } else {
                bf16x8 z = {};
                a[s] = z;
            }
        }
    }
#pragma unroll 1
    for (int nt = 0; nt < R / 32; ++nt) {
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
            if (m < QH) qt[m * R + n] = f32_to_bf16_rne(acc[r]);
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

template <int R>
hipError_t launch_bf16_r(const void *q, const void *W, void *qt, int64_t QH, int d, hipStream_t s)
{
    const unsigned blocks = (unsigned)((QH + 127) / 128);
    const u16 *qq = (const u16 *)q;
    const u16 *ww = (const u16 *)W;
    u16 *oo = (u16 *)qt;
    switch (d) {
    case 32: hipLaunchKernelGGL((k_absorb_bf16<R, 32>), dim3(blocks), dim3(256), 0, s, qq, ww, oo, QH); break;
    case 64: hipLaunchKernelGGL((k_absorb_bf16<R, 64>), dim3(blocks), dim3(256), 0, s, qq, ww, oo, QH); break;
    case 128: hipLaunchKernelGGL((k_absorb_bf16<R, 128>), dim3(blocks), dim3(256), 0, s, qq, ww, oo, QH); break;
    case 256: hipLaunchKernelGGL((k_absorb_bf16<R, 256>), dim3(blocks), dim3(256), 0, s, qq, ww, oo, QH); break;
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

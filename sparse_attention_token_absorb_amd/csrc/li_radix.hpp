// Radix-selection primitives shared by the selection kernels and the
// filter pass fused into the decode scoring kernels (gfx950, wave64):
// a DPP prefix scan across a wave and the block-wide threshold-bin search
// on an LDS histogram.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace li {
namespace {

__device__ __forceinline__ uint64_t lanes_below() { return (1ull << (threadIdx.x & 63)) - 1ull; }

// Inclusive prefix sum over the lanes of a wave (lane 0 first), on DPP: row
// shifts by 1, 2, 4 and 8 inside each row of 16 lanes, then the last lane of
// row 0 (and of row 2) is added to row 1 (row 3), and that of row 1 to rows
// 2 and 3.  Lanes without a source read 0.  Whole waves must reach it.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x)
{
    int v = (int)x;
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false); // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false); // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false); // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false); // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false); // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false); // row_bcast:31 into rows 2, 3
    return (uint32_t)v;
}

// Block-wide search on an LDS histogram of NB bins (bin order = key order)
// for NR budgets at once: for budget j, sh.res[2j] = the bin b holding the
// rem[j]-th largest element (-1 if rem[j] exceeds the total) and
// sh.res[2j+1] = elements in bins > b (sh: LDS scratch with uint32_t
// wtot[T/64] and int res[4]).  Each thread sums a run of adjacent bins, a
// DPP scan and the wave totals give every thread the count above its run,
// and the thread whose run crosses a budget searches it.  Two barriers; the
// caller puts a barrier between its reads of an earlier result and the next
// call.
template <int T, int NB, int NR, class SH>
__device__ void find_bins(const uint32_t *h, const uint32_t (&rem)[NR], SH &sh)
{
    constexpr int NW = T / 64;
    constexpr int PER = NB >= T ? NB / T : 1; // bins per thread
    constexpr int ACT = NB / PER;             // threads holding bins
    static_assert(PER * ACT == NB && NR <= 2, "bins per thread");
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    uint32_t v[PER];
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        v[j] = tid < ACT ? h[tid * PER + j] : 0u;
        s += v[j];
    }
    // run of this thread and all later ones: the wave's suffix plus later waves
    const uint32_t p = wave_incl_scan(s);
    const uint32_t wtotal = (uint32_t)__builtin_amdgcn_readlane((int)p, 63);
    if (lane == 0) sh.wtot[wv] = wtotal;
    if (tid < NR) sh.res[2 * tid] = -1;
    __syncthreads();
    uint32_t later = 0;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) later += w2 > wv ? sh.wtot[w2] : 0u;
    const uint32_t incl = wtotal - p + s + later; // elements in this run and above it
    const uint32_t excl = incl - s;               // elements above this run
#pragma unroll
    for (int j = 0; j < NR; ++j) {
        if (excl < rem[j] && incl >= rem[j]) {
            uint32_t acc = excl;
#pragma unroll
            for (int jj = PER - 1; jj >= 0; --jj) {
                if (acc + v[jj] >= rem[j]) {
                    sh.res[2 * j] = tid * PER + jj;
                    sh.res[2 * j + 1] = (int)acc;
                    break;
                }
                acc += v[jj];
            }
        }
    }
    __syncthreads();
}

} // namespace
} // namespace li

// Anchor-side latent append (gfx950).
//
// LatentIndex (paperlayer.ai summary of arXiv:2610.04635), §3.1 and §B.2: the
// group's shared latent is cached once per group, written by the anchor
// layer; followers only read it.  New rows are copied bit-exactly into the
// paged pool: row t -> page block_table[seq[t]][pos[t] / 64], slot pos[t] % 64.
#include "li_internal.hpp"

namespace li {
namespace {

// One thread per 16-byte chunk of a row.  Rows whose sequence, position or
// page lies outside the cache are not written.
__global__ __launch_bounds__(256) void k_append(uint8_t *pool, const int32_t *bt, PoolGeom geo, int row_bytes,
                                                const uint8_t *rows, const int32_t *seq, const int32_t *pos, int T)
{
    const int chunks = row_bytes / 16;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)T * chunks) return;
    const int t = (int)(i / chunks);
    const int c = (int)(i % chunks);
    const int64_t slot = geo.slot(bt, seq[t], pos[t]);
    if (slot < 0) return;
    const uint4 v = *(const uint4 *)(rows + (int64_t)t * row_bytes + c * 16);
    *(uint4 *)(pool + slot * row_bytes + c * 16) = v;
}

// Rows whose size is not a multiple of 16 bytes (fp32 with odd r): 4 bytes per thread.
__global__ __launch_bounds__(256) void k_append4(uint8_t *pool, const int32_t *bt, PoolGeom geo, int row_bytes,
                                                 const uint8_t *rows, const int32_t *seq, const int32_t *pos, int T)
{
    const int words = row_bytes / 4;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)T * words) return;
    const int t = (int)(i / words);
    const int c = (int)(i % words);
    const int64_t slot = geo.slot(bt, seq[t], pos[t]);
    if (slot < 0) return;
    const uint32_t v = *(const uint32_t *)(rows + (int64_t)t * row_bytes + c * 4);
    *(uint32_t *)(pool + slot * row_bytes + c * 4) = v;
}

} // namespace

hipError_t launch_append(void *pool, const int32_t *bt, const PoolGeom &geo, int r, int esize, const void *rows,
                         const int32_t *seq, const int32_t *pos, int T, hipStream_t s)
{
    if (T <= 0) return hipSuccess;
    const int row_bytes = r * esize;
    if (row_bytes % 16 == 0) {
        const int64_t n = (int64_t)T * (row_bytes / 16);
        hipLaunchKernelGGL(k_append, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (uint8_t *)pool, bt, geo,
                           row_bytes, (const uint8_t *)rows, seq, pos, T);
    } else {
        const int64_t n = (int64_t)T * (row_bytes / 4);
        hipLaunchKernelGGL(k_append4, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (uint8_t *)pool, bt, geo,
                           row_bytes, (const uint8_t *)rows, seq, pos, T);
    }
    return hipGetLastError();
}

} // namespace li

// Internal definitions shared by the HIP translation units of liblatentindex.
// Target: gfx950 (MI355X, CDNA4), wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace li {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr int kPage = 64;        // rows per cache page
constexpr int kTile = 32;        // latent rows per MFMA column tile
constexpr int kWave = 64;
constexpr int kBlock = 256;      // threads per workgroup of every kernel here
constexpr int kDigit0Shift = 20; // first radix digit: key bits [31:20]

// Order-preserving map of an fp32 score to uint32 (larger score -> larger
// key).  -0.0 is folded onto +0.0 so equal scores give equal keys.
__device__ __forceinline__ uint32_t score_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u << 1) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Device-resident indices (sequence ids, page ids, positions, candidates)
// come from the caller's buffers and cannot be checked on the host; every
// kernel bounds them where it uses them, so an out-of-range value gives
// meaningless results but never an access outside the buffers.
__device__ __forceinline__ int clamp_index(int v, int n) { return v < 0 ? 0 : (v < n ? v : n - 1); }

// Rows a query scores: the causal prefix, inclusive of its own position,
// capped by the rows present in its sequence.
__device__ __forceinline__ int valid_rows(int pos, int seq_len)
{
    int n = pos + 1 < seq_len ? pos + 1 : seq_len;
    return n > 0 ? n : 0;
}

// Round-to-nearest-even fp32 -> bf16 bits.
__device__ __forceinline__ u16 f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (u16)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(u16 h) { return __uint_as_float(((uint32_t)h) << 16); }

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v)
{
    for (int off = 32; off > 0; off >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, off));
    return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off));
    return v;
}

// s_waitcnt immediate (gfx9 encoding) for vmcnt(N), other counters untouched.
template <int N>
struct VmcntImm {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    static constexpr int value = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
};

// Wait for vector-memory operations through the compiler's own waitcnt
// model (it then knows the wait happened), not through inline asm.
template <int N>
__device__ __forceinline__ void wait_vmcnt_known()
{
    __builtin_amdgcn_s_waitcnt(VmcntImm<N>::value);
}

// Wait until at most N vector-memory operations of this wave are in flight.
// The memory clobber keeps the compiler from moving LDS reads above it.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Per-query parameters of one selection problem ("virtual row" of scores).
//   key(i)  = score_key(S[q*ld + (gmap ? gmap[q*gld + i] : i)])
//   out(i)  = omap ? omap[q*old + i] : i
struct SelRow {
    const float *S;
    int64_t ld;
    const int32_t *gmap;
    int64_t gld;
    const int32_t *omap;
    int64_t old;
};

} // namespace li

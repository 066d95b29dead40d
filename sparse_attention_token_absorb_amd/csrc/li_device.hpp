// Device helpers shared by the scoring kernels (gfx950): LDS-typed
// pointers, LDS DMA, barriers and waits, and the fused score epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "li_common.hpp"
#include "li_internal.hpp"

namespace li {
namespace {

// LDS-typed pointers keep every access a ds_* instruction (a generic pointer
// would become a flat access that also waits on global memory).
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef const __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef const __attribute__((address_space(3))) float lds_f32;
typedef const __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) int32_t lds_i32;
typedef const __attribute__((address_space(4))) int32_t const_i32_t;

// 16 bytes per lane from global memory straight into LDS at
// lds_uniform + lane * 16 (global_load_lds_dwordx4, LDS base in M0).
// Written as inline asm on purpose: the compiler then does not know that
// LDS is being written, and does not drain every such load (vmcnt(0))
// before each later LDS read.  The kernels wait for these loads themselves
// (wait_after / wait_vmcnt, counting loads only: vector loads complete in
// issue order) and publish them to other waves with a barrier.  The
// instruction has no VGPR result, so no register is left in flight.  M0 is
// saved and restored around it (with the wait state a write of M0 needs
// before an LDS-direct load), so the compiler's own use of M0 is untouched.
__device__ __forceinline__ void dma16(const void *g, lds_u8 *lds_uniform)
{
    const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_uniform);
    uint32_t saved;
    asm volatile("s_mov_b32 %[sv], m0\n\t"
                 "s_mov_b32 m0, %[lds]\n\t"
                 "s_nop 0\n\t"
                 "global_load_lds_dwordx4 %[addr], off\n\t"
                 "s_nop 0\n\t"
                 "s_mov_b32 m0, %[sv]"
                 : [sv] "=&s"(saved)
                 : [addr] "v"(g), [lds] "s"(lds)
                 : "memory");
}

// dma16 with the non-temporal policy: the bytes are streamed through without
// being kept in L2 or the Infinity Cache, so a long one-pass read does not
// evict the lines that other data (the scores being written, the query)
// still needs.
__device__ __forceinline__ void dma16_nt(const void *g, lds_u8 *lds_uniform)
{
    const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_uniform);
    uint32_t saved;
    asm volatile("s_mov_b32 %[sv], m0\n\t"
                 "s_mov_b32 m0, %[lds]\n\t"
                 "s_nop 0\n\t"
                 "global_load_lds_dwordx4 %[addr], off nt\n\t"
                 "s_nop 0\n\t"
                 "s_mov_b32 m0, %[sv]"
                 : [sv] "=&s"(saved)
                 : [addr] "v"(g), [lds] "s"(lds)
                 : "memory");
}

template <bool NT>
__device__ __forceinline__ void dma16p(const void *g, lds_u8 *lds_uniform)
{
    if constexpr (NT)
        dma16_nt(g, lds_uniform);
    else
        dma16(g, lds_uniform);
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

// Wait until at most `after` * PER vector-memory operations are in flight
// (the count must be an immediate, hence the switch).
template <int PER, int MAXA>
__device__ __forceinline__ void wait_after(int after)
{
    static_assert(PER * MAXA < 64, "vmcnt range");
    switch (after) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<PER>(); break;
    case 2: wait_vmcnt<(MAXA >= 2 ? 2 : 1) * PER>(); break;
    case 3: wait_vmcnt<(MAXA >= 3 ? 3 : 1) * PER>(); break;
    case 4: wait_vmcnt<(MAXA >= 4 ? 4 : 1) * PER>(); break;
    case 5: wait_vmcnt<(MAXA >= 5 ? 5 : 1) * PER>(); break;
    case 6: wait_vmcnt<(MAXA >= 6 ? 6 : 1) * PER>(); break;
    default: wait_vmcnt<(MAXA >= 7 ? 7 : 1) * PER>(); break;
    }
}

// Wait until at most n (wave-uniform, 0 <= n <= 15) vector-memory
// operations of this wave are in flight.
__device__ __forceinline__ void wait_vmcnt_upto(int n)
{
    switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    default: wait_vmcnt<15>(); break;
    }
}

// 4 bytes per lane from global memory straight into LDS at
// lds_uniform + lane * 4 (global_load_lds_dword), issued like dma16.
__device__ __forceinline__ void dma4(const void *g, lds_u8 *lds_uniform)
{
    const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_uniform);
    uint32_t saved;
    asm volatile("s_mov_b32 %[sv], m0\n\t"
                 "s_mov_b32 m0, %[lds]\n\t"
                 "s_nop 0\n\t"
                 "global_load_lds_dword %[addr], off\n\t"
                 "s_nop 0\n\t"
                 "s_mov_b32 m0, %[sv]"
                 : [sv] "=&s"(saved)
                 : [addr] "v"(g), [lds] "s"(lds)
                 : "memory");
}

// f(std::integral_constant<int, i>{}) for i = 0 .. N-1 in order: a loop
// whose index is a compile-time constant in its body.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// A wave-uniform address held in an SGPR pair.
__device__ __forceinline__ uint64_t uniform_addr(const void *p)
{
    const uint64_t a = (uint64_t)(uintptr_t)p;
    return (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a) |
           ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32);
}

// dma16 and dma4 from a wave-uniform base address plus a per-lane 32-bit
// byte offset: the load unit forms each lane's address, so a caller whose
// lane offsets are fixed spends no vector instructions on addresses.  NT:
// the non-temporal policy of dma16_nt.
template <bool NT = false>
__device__ __forceinline__ void dma16s(const void *base_uniform, uint32_t off, lds_u8 *lds_uniform)
{
    const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_uniform);
    const uint64_t b = uniform_addr(base_uniform);
    uint32_t saved;
    if constexpr (NT) {
        asm volatile("s_mov_b32 %[sv], m0\n\t"
                     "s_mov_b32 m0, %[lds]\n\t"
                     "s_nop 0\n\t"
                     "global_load_lds_dwordx4 %[off], %[base] nt\n\t"
                     "s_nop 0\n\t"
                     "s_mov_b32 m0, %[sv]"
                     : [sv] "=&s"(saved)
                     : [off] "v"(off), [base] "s"(b), [lds] "s"(lds)
                     : "memory");
    } else {
        asm volatile("s_mov_b32 %[sv], m0\n\t"
                     "s_mov_b32 m0, %[lds]\n\t"
                     "s_nop 0\n\t"
                     "global_load_lds_dwordx4 %[off], %[base]\n\t"
                     "s_nop 0\n\t"
                     "s_mov_b32 m0, %[sv]"
                     : [sv] "=&s"(saved)
                     : [off] "v"(off), [base] "s"(b), [lds] "s"(lds)
                     : "memory");
    }
}

__device__ __forceinline__ void dma4s(const void *base_uniform, uint32_t off, lds_u8 *lds_uniform)
{
    const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_uniform);
    const uint64_t b = uniform_addr(base_uniform);
    uint32_t saved;
    asm volatile("s_mov_b32 %[sv], m0\n\t"
                 "s_mov_b32 m0, %[lds]\n\t"
                 "s_nop 0\n\t"
                 "global_load_lds_dword %[off], %[base]\n\t"
                 "s_nop 0\n\t"
                 "s_mov_b32 m0, %[sv]"
                 : [sv] "=&s"(saved)
                 : [off] "v"(off), [base] "s"(b), [lds] "s"(lds)
                 : "memory");
}

// max(x, 0) in one integer max on the bit pattern (negative floats, -0.0
// included, have the sign bit set and become +0.0).
// Raw buffer resources (gfx9 family): the fourth descriptor word of an
// untyped 32-bit buffer, and a byte offset past any buffer's record count.
// A raw buffer access whose offset is at or beyond the record count is
// dropped (a store writes nothing, a load returns 0), which lets a masked
// store go without a branch.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kBufferDrop = (int)0x80000000;

__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// ReLU, head weights and head sum: the score of tile row (lane % 32).
template <int HB>
__device__ __forceinline__ float epilogue(const f32x16 (&acc)[HB], const float (&w)[HB][16])
{
    float ps[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        ps[hb] = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) ps[hb] = fmaf(w[hb][r], relu(acc[hb][r]), ps[hb]);
    }
    float p = ps[0];
#pragma unroll
    for (int hb = 1; hb < HB; ++hb) p += ps[hb];
    // the two lane halves hold the two head halves of each row: swap halves
    // across the wave (a VALU permute; the results hold lane l%32's value and
    // lane l%32+32's, one each) and add
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(p), false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Multiplies the complex pair (re, im) by exp(i pos theta) in fp64: the
// phase as one product, then plain products and sums (no fused
// multiply-add), rounded as written.
__device__ __forceinline__ void rope_pair(double &re, double &im, int pos, double theta)
{
#pragma clang fp contract(off)
    const double ang = (double)pos * theta;
    double sn, cs;
    sincos(ang, &sn, &cs);
    const double a = re * cs - im * sn;
    const double b = re * sn + im * cs;
    re = a;
    im = b;
}

// x rounded to the nearest bf16 value (ties to even), returned as a float
// (finite x).
__device__ __forceinline__ float bf16_round(float x)
{
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return __uint_as_float(u & 0xFFFF0000u);
}

// MFMA operands that set a 32x32 accumulator block to the heads' biases:
// A_b row h (lanes 0..31) holds bias[h] split into three bf16 parts at
// k = 0..2 (exact: 8 + 8 + 8 significant bits), B_1 ones at k = 0..2 for
// every column, so v_mfma_f32_32x32x16_bf16(A_b, B_1, 0) gives bias[h] in
// every row of head h.  bias: the query's H values (null or !live: zeros).
template <int HB>
__device__ __forceinline__ void bias_operands(const float *bias, int H, bool live, bf16x8 (&ab)[HB], bf16x8 &bones)
{
    const int lane = threadIdx.x & 63;
    const bool lo_half = lane < 32;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        const int h = hb * 32 + (lane & 31);
        const float b = bias && lo_half && live && h < H ? bias[h] : 0.0f;
        const float hi = bf16_round(b);
        const float mid = bf16_round(b - hi);
        const float lo = bf16_round((b - hi) - mid);
        bf16x8 v = {};
        v[0] = (__bf16)hi;
        v[1] = (__bf16)mid;
        v[2] = (__bf16)lo;
        ab[hb] = v;
    }
    bf16x8 o = {};
    if (lo_half) {
        o[0] = (__bf16)1.0f;
        o[1] = (__bf16)1.0f;
        o[2] = (__bf16)1.0f;
    }
    bones = o;
}

// Adds each accumulator's head bias (b: the query's 64 staged biases, heads
// past H zero) before the ReLU; accumulator r of block hb holds head
// hb*32 + (r/4)*8 + (lane/32)*4 + r%4 of tile row lane % 32.
template <int HB>
__device__ __forceinline__ void add_bias(f32x16 (&acc)[HB], const lds_f32 *b)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 v = *(lds_f32x4 *)(b + hb * 32 + g * 8 + (lane >> 5) * 4);
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[hb][g * 4 + t] += v[t];
        }
}

__device__ __forceinline__ void hist_zero(uint32_t *h, int nthreads, int tid)
{
    for (int i = tid; i < kHistBins; i += nthreads) h[i] = 0;
}

__device__ __forceinline__ void hist_flush(const uint32_t *h, int32_t *g, int nthreads, int tid)
{
    for (int i = tid; i < kHistBins; i += nthreads)
        if (h[i]) atomicAdd(&g[i], (int)h[i]);
}

} // namespace
} // namespace li

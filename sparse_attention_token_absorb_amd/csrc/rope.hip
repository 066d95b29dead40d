// RoPE-compatible structured decoder (gfx950).
//
// LatentIndex (paperlayer.ai summary of arXiv:2610.04635), §A.2: the rotary
// sources of the shared latent share the native rotary phase, so the latent
// is rotated once, when it is cached, and each layer's decoder is absorbed
// into its post-RoPE query; §A.4: per rotary frequency, layer-specific
// complex decoder coefficients over shared complex sources; §A.3: a dense
// NoPE decoder with an output bias; §3.1: a latent row is its rotary part
// followed by its NoPE part, kept once for the whole group.
//
//   append   rotary pair j of a row at position p turns by p * theta_(j % F)
//            (fp64), the row is rounded once to the pool dtype;
//   decoder  the complex coefficients become 2x2 blocks of a dense W, so the
//            ordinary absorption GEMM computes q_f * conj(D[f][s]) for every
//            (source, frequency) slot next to the NoPE product;
//   bias     b = q_nope . beta per (query, head), summed in fp64.
#include "li_device.hpp"
#include "li_internal.hpp"

namespace li {
namespace {

// fp64 -> bf16 bits, round to nearest even, in one step (finite values).
__device__ __forceinline__ u16 f64_to_bf16_rne(double x)
{
    int e;
    const double m = frexp(x, &e); // x = m 2^e, |m| in [0.5, 1)
    const double v = ldexp(rint(ldexp(m, 8)), e - 8); // 8 significant bits; rint ties to even
    return (u16)(__float_as_uint((float)v) >> 16);  // exact in fp32
}

template <bool BF16>
__device__ __forceinline__ double load_elem(const void *p, int64_t i)
{
    if constexpr (BF16) return (double)bf16_to_f32(((const u16 *)p)[i]);
    else return (double)((const float *)p)[i];
}

template <bool BF16>
__device__ __forceinline__ void store_elem(void *p, int64_t i, double v)
{
    if constexpr (BF16) ((u16 *)p)[i] = f64_to_bf16_rne(v);
    else ((float *)p)[i] = (float)v;
}

// One thread per element pair of a row (a last unpaired element of an odd
// fp32 row is copied).
template <bool BF16>
__global__ __launch_bounds__(256) void k_append_rope(void *pool, const int32_t *bt, PoolGeom geo, int r,
                                                     const void *rows, const int32_t *seq, const int32_t *pos, int T,
                                                     const RopeArgs rope)
{
    const int pairs = (r + 1) / 2;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)T * pairs) return;
    const int t = (int)(i / pairs);
    const int j = (int)(i % pairs);
    const int p = pos[t];
    const int64_t slot = geo.slot(bt, seq[t], p);
    if (slot < 0) return; // a sequence, position or page outside the cache: the row is not written
    const int64_t dst = slot * r;
    const int64_t src = (int64_t)t * r;
    double re = load_elem<BF16>(rows, src + 2 * j);
    if (2 * j + 1 >= r) {
        store_elem<BF16>(pool, dst + 2 * j, re);
        return;
    }
    double im = load_elem<BF16>(rows, src + 2 * j + 1);
    if (j < rope.S * rope.F) rope_pair(re, im, p, rope.theta[j % rope.F]);
    store_elem<BF16>(pool, dst + 2 * j, re);
    store_elem<BF16>(pool, dst + 2 * j + 1, im);
}

// w_dec [d][r] from D [F][S][2] and Wn [d_nope][r_nope], one thread per
// entry.  For slot j = s F + f, with q_f = a + i b and D[f][s] = c + i e,
//   qt[2j]   = a c + b e   : W[2f][2j]   = c,  W[2f+1][2j]   = e
//   qt[2j+1] = b c - a e   : W[2f][2j+1] = -e, W[2f+1][2j+1] = c.
template <bool BF16>
__global__ __launch_bounds__(256) void k_rope_decoder(const void *D, const void *Wn, int F, int S, int d_nope,
                                                      int r_nope, void *W)
{
    const int d = 2 * F + d_nope, r = 2 * S * F + r_nope;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)d * r) return;
    const int e = (int)(i / r), t = (int)(i % r);
    // bits of the value as stored (bf16: 16 bits; fp32: 32 bits); negation flips the sign bit
    const uint32_t sign = BF16 ? 0x8000u : 0x80000000u;
    auto get = [&](const void *p, int64_t k) -> uint32_t {
        if constexpr (BF16) return ((const u16 *)p)[k];
        else return __float_as_uint(((const float *)p)[k]);
    };
    uint32_t v = 0;
    if (e < 2 * F && t < 2 * S * F) {
        const int f = e >> 1, jj = t >> 1;
        if (jj % F == f) {
            const int s = jj / F;
            const uint32_t c = get(D, ((int64_t)f * S + s) * 2), ei = get(D, ((int64_t)f * S + s) * 2 + 1);
            const bool row_re = (e & 1) == 0, col_re = (t & 1) == 0;
            v = row_re ? (col_re ? c : ei ^ sign) : (col_re ? ei : c);
        }
    } else if (e >= 2 * F && t >= 2 * S * F) {
        v = get(Wn, (int64_t)(e - 2 * F) * r_nope + (t - 2 * S * F));
    }
    if constexpr (BF16) ((u16 *)W)[i] = (u16)v;
    else ((float *)W)[i] = __uint_as_float(v);
}

// bias[i] = sum_e q[i][d_rope + e] beta[e]: every product is exact in fp64
// (bf16 or fp32 times fp32), summed in fp64 and rounded once.
template <bool BF16>
__global__ __launch_bounds__(256) void k_query_bias(const void *q, const float *beta, int64_t QH, int d, int d_rope,
                                                    float *bias)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= QH) return;
    double acc = 0.0;
    for (int e = 0; e < d - d_rope; ++e) acc += load_elem<BF16>(q, i * d + d_rope + e) * (double)beta[e];
    bias[i] = (float)acc;
}

} // namespace

hipError_t launch_append_rope(void *pool, const int32_t *bt, const PoolGeom &geo, int r, int esize, const void *rows,
                              const int32_t *seq, const int32_t *pos, int T, const RopeArgs &rope, hipStream_t s)
{
    if (T <= 0) return hipSuccess;
    const int64_t n = (int64_t)T * ((r + 1) / 2);
    const dim3 grid((unsigned)((n + 255) / 256));
    if (esize == 2)
        hipLaunchKernelGGL(k_append_rope<true>, grid, dim3(256), 0, s, pool, bt, geo, r, rows, seq, pos, T,
                           rope);
    else
        hipLaunchKernelGGL(k_append_rope<false>, grid, dim3(256), 0, s, pool, bt, geo, r, rows, seq, pos, T,
                           rope);
    return hipGetLastError();
}

hipError_t launch_rope_decoder(const void *D, const void *Wn, int F, int S, int d_nope, int r_nope, void *W, int esize,
                               hipStream_t s)
{
    const int64_t n = (int64_t)(2 * F + d_nope) * (2 * S * F + r_nope);
    if (n <= 0) return hipSuccess;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (esize == 2)
        hipLaunchKernelGGL(k_rope_decoder<true>, grid, dim3(256), 0, s, D, Wn, F, S, d_nope, r_nope, W);
    else
        hipLaunchKernelGGL(k_rope_decoder<false>, grid, dim3(256), 0, s, D, Wn, F, S, d_nope, r_nope, W);
    return hipGetLastError();
}

hipError_t launch_query_bias(const void *q, const float *beta, int64_t QH, int d, int d_rope, float *bias, bool bf16,
                             hipStream_t s)
{
    if (QH <= 0) return hipSuccess;
    const dim3 grid((unsigned)((QH + 255) / 256));
    if (bf16)
        hipLaunchKernelGGL(k_query_bias<true>, grid, dim3(256), 0, s, q, beta, QH, d, d_rope, bias);
    else
        hipLaunchKernelGGL(k_query_bias<false>, grid, dim3(256), 0, s, q, beta, QH, d, d_rope, bias);
    return hipGetLastError();
}

} // namespace li

// C ABI of liblatentindex: argument validation, workspace carving and
// kernel dispatch.  Every entry point validates on the host first and only
// then enqueues work on the caller's stream; nothing here allocates, frees
// or synchronizes.
#include <stdarg.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include <math.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>

#include "../../include/latentindex.h"
#include "li_internal.hpp"
#include "li_timing.hpp"
#include "li_probe.hpp"

// Scratch of li_score_topk_noalloc (the workspace of li_score_topk): one copy
// per GPU, held until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory; the device address of each GPU's
// copy comes from hipGetSymbolAddress and is the only form of it that is
// passed to kernels.
static constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

thread_local std::string g_last_error;

li_status fail(li_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
li_status fail(li_status s, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

li_status ok()
{
    g_last_error.clear();
    return LI_OK;
}

li_status hip_fail(hipError_t e, const char *where)
{
    return fail(LI_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

int64_t score_ld(int32_t max_valid) { return ((int64_t)std::max(max_valid, 1) + 63) / 64 * 64; }

bool r_supported(int32_t r, li_dtype dt)
{
    if (dt == LI_BF16) return r == 64 || r == 128 || r == 256;
    if (dt == LI_FP32) return r >= 1 && r <= 256;
    if (dt == LI_FP8) return r == 128 || r == 256;
    return false;
}

li_status check_cache(const li_cache *c)
{
    if (!c) return fail(LI_ERR_NULL, "cache descriptor is NULL");
    if (!c->pool || !c->block_table || !c->seq_lens) return fail(LI_ERR_NULL, "cache pool/block_table/seq_lens is NULL");
    if (c->page_size != LI_PAGE_SIZE) return fail(LI_ERR_UNSUPPORTED, "page_size %d (only %d)", c->page_size, LI_PAGE_SIZE);
    if (c->batch <= 0 || c->max_pages <= 0 || c->num_pages <= 0)
        return fail(LI_ERR_SHAPE, "batch %d, max_pages %d, num_pages %d must be positive", c->batch, c->max_pages,
                    c->num_pages);
    if (c->dtype != LI_BF16 && c->dtype != LI_FP32 && c->dtype != LI_FP8)
        return fail(LI_ERR_UNSUPPORTED, "dtype %d", (int)c->dtype);
    if (!r_supported(c->r, c->dtype)) return fail(LI_ERR_UNSUPPORTED, "latent width r=%d for dtype %d", c->r, (int)c->dtype);
    if (c->dtype == LI_FP8 && !c->scales) return fail(LI_ERR_NULL, "FP8 cache without scales");
    return LI_OK;
}

li_status check_queries(const li_queries *qs, const li_cache *c)
{
    if (!qs) return fail(LI_ERR_NULL, "queries descriptor is NULL");
    if (qs->Q < 0) return fail(LI_ERR_SHAPE, "Q=%d", qs->Q);
    if (qs->Q > 0 && (!qs->seq || !qs->pos)) return fail(LI_ERR_NULL, "queries seq/pos is NULL");
    if (qs->max_valid < 0 || (int64_t)qs->max_valid > (int64_t)c->max_pages * LI_PAGE_SIZE)
        return fail(LI_ERR_SHAPE, "max_valid=%d outside [0, max_pages*%d]", qs->max_valid, LI_PAGE_SIZE);
    return LI_OK;
}

// Validates a rotary layout against a latent width and fills the kernel's
// copy, with each frequency's phase step theta_f = base^(-2f / (2F)) in fp64.
li_status rope_args(const li_rope *rope, int32_t r, li::RopeArgs *out)
{
    if (!rope) return fail(LI_ERR_NULL, "rope descriptor is NULL");
    if (rope->freqs < 1 || rope->freqs > li::kMaxRopeFreqs || rope->sources < 1)
        return fail(LI_ERR_SHAPE, "rope freqs=%d (1..%d), sources=%d (>= 1)", rope->freqs, li::kMaxRopeFreqs,
                    rope->sources);
    if ((int64_t)2 * rope->sources * rope->freqs > r)
        return fail(LI_ERR_SHAPE, "2 * sources * freqs = %lld exceeds r=%d", (long long)2 * rope->sources * rope->freqs,
                    r);
    if (!(rope->base > 1.0) || !isfinite(rope->base)) return fail(LI_ERR_SHAPE, "rope base %g must be > 1", rope->base);
    *out = li::RopeArgs{};
    out->F = rope->freqs;
    out->S = rope->sources;
    for (int f = 0; f < rope->freqs; ++f)
        out->theta[f] = pow(rope->base, -(double)(2 * f) / (double)(2 * rope->freqs));
    return LI_OK;
}

// Whether a decode scoring launch reads its latent rows with the
// non-temporal policy.  A group's layers score the same latent one after the
// other, so while the rows fit the 256 MB last-level cache (Infinity Cache)
// with room to spare, letting them stay there serves the next layer; a launch
// that streams half of that cache or more would mostly evict other data.
// Measured: the 132 MiB FP8 latent of four 131072-row sequences scores 7%
// faster from HBM (cold) and no slower warm when streamed non-temporally,
// and a per-layer indexer's 128 MiB key caches (four layers in turn) 7%
// faster per layer.
// LI_STREAM_NT=0|1 overrides (read once).
constexpr int64_t kStreamNtBytes = 128ll << 20;

bool stream_nt(int64_t bytes)
{
    static const int over = [] {
        const char *e = getenv("LI_STREAM_NT");
        if (e && strcmp(e, "0") == 0) return 0;
        if (e && strcmp(e, "1") == 0) return 1;
        return -1;
    }();
    if (over >= 0) return over == 1;
    return bytes >= kStreamNtBytes;
}

// Where the filter pass of long-row decode selection runs (li_fused_filter):
// 0 its own kernel, 1 inside the scoring kernel when its grid is resident at
// once (see li::FilterArgs), 2 as 1 with a wait that always runs out.
std::atomic<int> g_fused_filter{-1};

int fused_filter_mode()
{
    int m = g_fused_filter.load(std::memory_order_relaxed);
    if (m < 0) {
        const char *e = getenv("LI_FUSED_FILTER");
        int init = e && strcmp(e, "0") == 0 ? 0 : 1;
        g_fused_filter.compare_exchange_strong(m, init);
        m = g_fused_filter.load(std::memory_order_relaxed);
    }
    return m;
}

// The fused pass's bound on its wait: 1 ms of the 100 MHz constant clock.
constexpr uint32_t kFilterWaitTicks = 100000;

li::ScoreArgs score_args(const li_cache *c, const li_queries *qs, const void *qt, const float *w, int32_t H)
{
    li::ScoreArgs a{};
    a.pool = c->pool;
    a.bt = c->block_table;
    a.max_pages = c->max_pages;
    a.num_pages = c->num_pages;
    a.batch = c->batch;
    a.seq_lens = c->seq_lens;
    a.qseq = qs->seq;
    a.qpos = qs->pos;
    a.qt = qt;
    a.w = w;
    a.H = H;
    a.Q = qs->Q;
    return a;
}

} // namespace

extern "C" {

static_assert(li::kSyncBytes == ((size_t)LI_WORKSPACE_ZEROED_BYTES + 255) / 256 * 256, "zeroed region size");

int32_t li_abi_version(void) { return LI_ABI_VERSION; }

const char *li_last_error(void) { return g_last_error.c_str(); }

const char *li_status_str(li_status s)
{
    switch (s) {
    case LI_OK: return "LI_OK";
    case LI_ERR_NULL: return "LI_ERR_NULL";
    case LI_ERR_SHAPE: return "LI_ERR_SHAPE";
    case LI_ERR_UNSUPPORTED: return "LI_ERR_UNSUPPORTED";
    case LI_ERR_WORKSPACE: return "LI_ERR_WORKSPACE";
    case LI_ERR_HIP: return "LI_ERR_HIP";
    }
    return "LI_ERR_UNKNOWN";
}

size_t li_workspace_bytes(int op, int32_t Q, int32_t max_valid, int32_t H, int32_t r, int32_t k, int32_t M)
{
    (void)H;
    (void)r;
    if (Q < 0 || k <= 0 || k > LI_MAX_TOPK) return 0;
    switch (op) {
    case LI_OP_SCORE_TOPK:
    case LI_OP_SCORE_TOPK_EXT_SCORES: {
        if (max_valid < 0) return 0;
        size_t b = op == LI_OP_SCORE_TOPK ? align256((size_t)Q * score_ld(max_valid) * 4) : 0;
        return li::kSyncBytes + b + align256(li::sel_workspace_bytes(Q, std::max(max_valid, 1)));
    }
    case LI_OP_HS_SELECT:
        if (M <= 0 || M > LI_MAX_TOPK) return 0;
        return li::kSyncBytes + align256((size_t)Q * M * 4) + align256(li::sel_workspace_bytes(Q, M));
    default: return 0;
    }
}

namespace {

li_status append_common(const li_cache *cache, const void *rows, const int32_t *seq, const int32_t *pos, int32_t T,
                        const li_rope *rope, hipStream_t stream)
{
    li_status st = check_cache(cache);
    if (st != LI_OK) return st;
    if (T < 0) return fail(LI_ERR_SHAPE, "T=%d", T);
    li::RopeArgs ra{};
    if (rope) {
        st = rope_args(rope, cache->r, &ra);
        if (st != LI_OK) return st;
    }
    if (T == 0) return ok();
    if (!rows || !seq || !pos) return fail(LI_ERR_NULL, "rows/seq/pos is NULL");
    const int esize = cache->dtype == LI_BF16 ? 2 : 4;
    hipError_t e;
    {
        li::TimedScope ts(LI_KERNEL_APPEND, stream);
        const li::PoolGeom geo{cache->batch, cache->max_pages, cache->num_pages};
        if (cache->dtype == LI_FP8)
            e = li::launch_append_fp8(cache->pool, cache->scales, cache->block_table, geo, cache->r, rows, seq, pos, T,
                                      ra, stream);
        else if (rope)
            e = li::launch_append_rope(cache->pool, cache->block_table, geo, cache->r, esize, rows, seq, pos, T, ra,
                                       stream);
        else
            e = li::launch_append(cache->pool, cache->block_table, geo, cache->r, esize, rows, seq, pos, T, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "append_latent launch");
    return ok();
}

} // namespace

li_status li_append_latent(const li_cache *cache, const void *rows, const int32_t *seq, const int32_t *pos, int32_t T,
                           hipStream_t stream)
{
    return append_common(cache, rows, seq, pos, T, nullptr, stream);
}

li_status li_append_latent_rope(const li_cache *cache, const void *rows, const int32_t *seq, const int32_t *pos,
                                int32_t T, const li_rope *rope, hipStream_t stream)
{
    if (!rope) return fail(LI_ERR_NULL, "rope descriptor is NULL");
    return append_common(cache, rows, seq, pos, T, rope, stream);
}

li_status li_rope_decoder(const void *D, const void *w_nope, const li_rope *rope, int32_t d_nope, int32_t r_nope,
                          void *w_dec, li_dtype dtype, hipStream_t stream)
{
    if (!rope) return fail(LI_ERR_NULL, "rope descriptor is NULL");
    if (rope->freqs < 1 || rope->freqs > li::kMaxRopeFreqs || rope->sources < 1)
        return fail(LI_ERR_SHAPE, "rope freqs=%d (1..%d), sources=%d (>= 1)", rope->freqs, li::kMaxRopeFreqs,
                    rope->sources);
    if (d_nope < 0 || r_nope < 0) return fail(LI_ERR_SHAPE, "d_nope=%d, r_nope=%d", d_nope, r_nope);
    if (dtype != LI_BF16 && dtype != LI_FP32) return fail(LI_ERR_UNSUPPORTED, "decoder dtype %d", (int)dtype);
    if (!D || !w_dec || (d_nope > 0 && r_nope > 0 && !w_nope)) return fail(LI_ERR_NULL, "D/w_nope/w_dec is NULL");
    hipError_t e = li::launch_rope_decoder(D, w_nope, rope->freqs, rope->sources, d_nope, r_nope, w_dec,
                                           dtype == LI_BF16 ? 2 : 4, stream);
    if (e != hipSuccess) return hip_fail(e, "rope_decoder launch");
    return ok();
}

li_status li_query_bias(const void *q, const float *beta, int32_t Q, int32_t H, int32_t d, int32_t d_rope, float *bias,
                        li_dtype dtype, hipStream_t stream)
{
    if (Q < 0 || H <= 0 || d <= 0 || d_rope < 0 || d_rope > d)
        return fail(LI_ERR_SHAPE, "Q=%d H=%d d=%d d_rope=%d", Q, H, d, d_rope);
    if (dtype != LI_BF16 && dtype != LI_FP32) return fail(LI_ERR_UNSUPPORTED, "query dtype %d", (int)dtype);
    if (Q == 0) return ok();
    if (!q || !bias || (d > d_rope && !beta)) return fail(LI_ERR_NULL, "q/beta/bias is NULL");
    hipError_t e = li::launch_query_bias(q, beta, (int64_t)Q * H, d, d_rope, bias, dtype == LI_BF16, stream);
    if (e != hipSuccess) return hip_fail(e, "query_bias launch");
    return ok();
}

li_status li_absorb_query(const void *q, const void *w_dec, void *q_tilde, int32_t Q, int32_t H, int32_t d, int32_t r,
                          li_dtype dtype, hipStream_t stream)
{
    if (Q < 0) return fail(LI_ERR_SHAPE, "Q=%d", Q);
    if (H <= 0 || H > LI_MAX_HEADS) return fail(LI_ERR_SHAPE, "H=%d outside [1, %d]", H, LI_MAX_HEADS);
    if (dtype != LI_BF16 && dtype != LI_FP32 && dtype != LI_FP8) return fail(LI_ERR_UNSUPPORTED, "dtype %d", (int)dtype);
    if (!r_supported(r, dtype)) return fail(LI_ERR_UNSUPPORTED, "r=%d for dtype %d", r, (int)dtype);
    if (dtype != LI_FP32 && d != 32 && d != 64 && d != 128 && d != 256)
        return fail(LI_ERR_UNSUPPORTED, "bf16 absorption needs d in {32,64,128,256}, got %d", d);
    if (dtype == LI_FP32 && (d <= 0 || d > 1024)) return fail(LI_ERR_SHAPE, "d=%d outside [1, 1024]", d);
    if (!w_dec && dtype != LI_FP8) return fail(LI_ERR_NULL, "w_dec is NULL (only LI_FP8 takes no decoder)");
    if (!w_dec && d != r) return fail(LI_ERR_SHAPE, "without a decoder d (%d) must equal r (%d)", d, r);
    if (Q == 0) return ok();
    if (!q || !q_tilde) return fail(LI_ERR_NULL, "q/q_tilde is NULL");
    hipError_t e;
    {
        li::TimedScope ts(LI_KERNEL_ABSORB, stream);
        if (dtype == LI_FP8)
            e = li::launch_absorb_fp8(q, w_dec, q_tilde, (int64_t)Q * H, d, r, stream);
        else
            e = li::launch_absorb(q, w_dec, q_tilde, (int64_t)Q * H, d, r, dtype == LI_BF16, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "absorb_query launch");
    return ok();
}

namespace {

li_status score_topk_impl(const li_cache *cache, const li_queries *queries, const void *q_tilde, const float *w,
                          const float *bias, int32_t H, int32_t k, int32_t *idx, int32_t *count, int32_t k_inner,
                          int32_t *idx_inner, int32_t *count_inner, float *scores, int64_t ld, void *ws,
                          size_t ws_bytes, hipStream_t stream)
{
    li_status st = check_cache(cache);
    if (st != LI_OK) return st;
    st = check_queries(queries, cache);
    if (st != LI_OK) return st;
    if (H <= 0 || H > LI_MAX_HEADS) return fail(LI_ERR_SHAPE, "H=%d outside [1, %d]", H, LI_MAX_HEADS);
    if (k <= 0 || k > LI_MAX_TOPK) return fail(LI_ERR_SHAPE, "k=%d outside [1, %d]", k, LI_MAX_TOPK);
    if (k_inner < 0 || k_inner > k) return fail(LI_ERR_SHAPE, "k_inner=%d outside [0, k=%d]", k_inner, k);
    const int32_t Q = queries->Q;
    if (Q == 0) return ok();
    if (!q_tilde || !w || !idx || !count) return fail(LI_ERR_NULL, "q_tilde/w/idx/count is NULL");
    if (k_inner > 0 && (!idx_inner || !count_inner)) return fail(LI_ERR_NULL, "idx_inner/count_inner is NULL");
    if (scores && ld < queries->max_valid) return fail(LI_ERR_SHAPE, "ld=%lld < max_valid=%d", (long long)ld, queries->max_valid);
    const int op = scores ? LI_OP_SCORE_TOPK_EXT_SCORES : LI_OP_SCORE_TOPK;
    const size_t need = li_workspace_bytes(op, Q, queries->max_valid, H, cache->r, k, 0);
    if (!ws || ws_bytes < need)
        return fail(LI_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : (size_t)0, need);

    int32_t *sync = (int32_t *)ws; // the zeroed region (see li_workspace_bytes)
    uint8_t *p = (uint8_t *)ws + li::kSyncBytes;
    float *S = scores;
    int64_t sld = ld;
    if (!S) {
        S = (float *)p;
        sld = score_ld(queries->max_valid);
        p += align256((size_t)Q * sld * 4);
    }
    const int64_t max_n = std::max(queries->max_valid, 1);
    li::SelWorkspace sw = li::sel_workspace_carve(p, Q, max_n, sync);

    li::SelCall sc{};
    sc.row = li::SelRow{S, sld, nullptr, 0, nullptr, 0};
    sc.src_mode = li::kSrcCausal;
    sc.qseq = queries->seq;
    sc.qpos = queries->pos;
    sc.seq_lens = cache->seq_lens;
    sc.batch = cache->batch;
    sc.Q = Q;
    sc.k = k;
    sc.max_n = queries->max_valid; // rows past the caller's bound are never scored
    sc.idx = idx;
    sc.count = count;
    // HS anchor: its own top-k_inner inside its top-k (a subset by construction)
    sc.k_inner = k_inner;
    sc.idx_inner = idx_inner;
    sc.count_inner = count_inner;

    const bool many = Q >= 4 * cache->batch;
    const bool scored = queries->max_valid > 0;
    // Decode scoring over rows longer than 8192 counts the first radix digit
    // as it writes (the row is read once more by selection anyway); over
    // shorter rows the one-workgroup selection counts the keys it holds, which
    // saves the histogram-clearing kernel; prefill scoring is MFMA-bound and
    // leaves the count to the selection pass.
    const bool fp8 = cache->dtype == LI_FP8;
    const bool fused_hist = scored && !(many && (cache->dtype == LI_BF16 || fp8)) &&
                            li::selection_wants_counts(Q, queries->max_valid);
    // On the filter path the histogram lives in the workspace's zeroed region
    // (no clearing kernel); the other counting paths clear theirs first.
    const bool filter_path = fused_hist && li::selection_filters(Q, queries->max_valid);
    hipError_t e = hipSuccess;
    bool filtered = false;
    if (scored) {
        if (fused_hist && !filter_path) {
            li::TimedScope ts(LI_KERNEL_SELECT, stream);
            e = li::launch_hist_clear(sw, Q, stream);
        }
        if (e != hipSuccess) return hip_fail(e, "histogram clear");
        li::ScoreArgs a = score_args(cache, queries, q_tilde, w, H);
        a.bias = bias;
        a.out = S;
        a.out_ld = sld;
        a.max_rows = queries->max_valid;
        a.hist = fused_hist ? sw.hist : nullptr;
        const int64_t row_bytes = fp8 ? cache->r + cache->r / 128 * 4 : (int64_t)cache->r * (cache->dtype == LI_BF16 ? 2 : 4);
        a.stream_nt = !many && stream_nt((int64_t)Q * queries->max_valid * row_bytes);
        // the selection's filter pass, offered to the scoring kernel
        const int fmode = fused_filter_mode();
        a.flt = li::FilterArgs{filter_path && fmode > 0, filter_path, k, k_inner, idx, idx_inner, sw.cand, sw.cand2,
                               sw.cap, fmode == 2 ? 0u : kFilterWaitTicks};
        li::TimedScope ts(many ? LI_KERNEL_SCORE_PREFILL : LI_KERNEL_SCORE_DECODE, stream, true);
        if (fp8)
            e = li::launch_score_fp8(a, cache->scales, li::fp8_query_scale_offset(Q, H, cache->r), cache->r, many,
                                     queries->max_valid, stream, &filtered);
        else
            e = li::launch_score(a, cache->r, cache->dtype == LI_BF16, many, queries->max_valid, stream, &filtered);
        if (e != hipSuccess) return hip_fail(e, "score launch");
    }
    {
        li::TimedScope ts(LI_KERNEL_SELECT, stream);
        e = li::launch_select(sc, sw, fused_hist, stream, filtered);
    }
    if (e != hipSuccess) return hip_fail(e, "select launch");

    return ok();
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];

// The current device's copy of the scratch array (resolved on the first call
// on that device, with the device current).
li_status scratch_on_current_device(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(LI_ERR_UNSUPPORTED, "device %d outside [0, %d)", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(LI_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return LI_OK;
}

} // namespace

li_status li_score_topk(const li_cache *cache, const li_queries *queries, const void *q_tilde, const float *w,
                        const float *bias, int32_t H, int32_t k, int32_t *idx, int32_t *count, int32_t k_inner,
                        int32_t *idx_inner, int32_t *count_inner, float *scores, int64_t ld, void *ws,
                        size_t ws_bytes, hipStream_t stream)
{
    return score_topk_impl(cache, queries, q_tilde, w, bias, H, k, idx, count, k_inner, idx_inner, count_inner,
                           scores, ld, ws, ws_bytes, stream);
}

li_status li_score_topk_noalloc(const li_cache *cache, const li_queries *queries, const void *q_tilde, const float *w,
                                const float *bias, int32_t H, int32_t k, int32_t *idx, int32_t *count,
                                int32_t k_inner, int32_t *idx_inner, int32_t *count_inner, float *scores, int64_t ld,
                                hipStream_t stream)
{
    li_status st = check_cache(cache);
    if (st != LI_OK) return st;
    st = check_queries(queries, cache);
    if (st != LI_OK) return st;
    if (k <= 0 || k > LI_MAX_TOPK) return fail(LI_ERR_SHAPE, "k=%d outside [1, %d]", k, LI_MAX_TOPK);
    if (queries->Q == 0) return ok();
    const int op = scores ? LI_OP_SCORE_TOPK_EXT_SCORES : LI_OP_SCORE_TOPK;
    const size_t need = li_workspace_bytes(op, queries->Q, queries->max_valid, H, cache->r, k, 0);
    if (need > kScratchBytes)
        return fail(LI_ERR_WORKSPACE,
                    "li_score_topk_noalloc needs %zu bytes of scratch at Q=%d, max_valid=%d, more than its %zu%s", need,
                    queries->Q, queries->max_valid, kScratchBytes, scores ? "" : " (a caller score buffer needs less)");
    void *ws = nullptr;
    st = scratch_on_current_device(&ws);
    if (st != LI_OK) return st;
    return score_topk_impl(cache, queries, q_tilde, w, bias, H, k, idx, count, k_inner, idx_inner, count_inner, scores,
                           ld, ws, kScratchBytes, stream);
}

li_status li_hs_select(const li_cache *cache, const li_queries *queries, const int32_t *cand,
                       const int32_t *cand_count, int32_t M, const void *q_tilde, const float *w, const float *bias,
                       int32_t H, int32_t k,
                       int32_t *idx, int32_t *count, float *cand_scores, void *ws, size_t ws_bytes,
                       hipStream_t stream)
{
    li_status st = check_cache(cache);
    if (st != LI_OK) return st;
    st = check_queries(queries, cache);
    if (st != LI_OK) return st;
    if (H <= 0 || H > LI_MAX_HEADS) return fail(LI_ERR_SHAPE, "H=%d outside [1, %d]", H, LI_MAX_HEADS);
    if (k <= 0 || k > LI_MAX_TOPK) return fail(LI_ERR_SHAPE, "k=%d outside [1, %d]", k, LI_MAX_TOPK);
    if (M <= 0 || M > LI_MAX_TOPK) return fail(LI_ERR_SHAPE, "M=%d outside [1, %d]", M, LI_MAX_TOPK);
    const int32_t Q = queries->Q;
    if (Q == 0) return ok();
    if (!cand || !cand_count || !q_tilde || !w || !idx || !count)
        return fail(LI_ERR_NULL, "cand/cand_count/q_tilde/w/idx/count is NULL");
    const size_t need = li_workspace_bytes(LI_OP_HS_SELECT, Q, 0, H, cache->r, k, M);
    if (!ws || ws_bytes < need)
        return fail(LI_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : (size_t)0, need);

    int32_t *sync = (int32_t *)ws; // the zeroed region (see li_workspace_bytes)
    uint8_t *p = (uint8_t *)ws + li::kSyncBytes;
    float *S = cand_scores ? cand_scores : (float *)p;
    float *S_pos = (float *)p; // by-position scores (see below)
    p += align256((size_t)Q * M * 4);
    li::SelWorkspace sw = li::sel_workspace_carve(p, Q, M, sync);

    // When M >= max_valid, no query has more valid rows than M, so scoring a
    // query's whole valid prefix reads no more rows than its candidates may
    // number, and reads them as contiguous tiles instead of through the
    // candidate -> page -> row chain.  The scores are then kept by position
    // (S_pos[q][row], stride M) and the selection reads each candidate's
    // score through the candidate list, which is exact for any list of
    // valid rows.
    if (queries->max_valid <= M) {
        hipError_t e = hipSuccess;
        li::ScoreArgs a = score_args(cache, queries, q_tilde, w, H);
        a.bias = bias;
        a.out = S_pos;
        a.out_ld = M;
        a.max_rows = queries->max_valid;
        a.hist = nullptr;
        const bool fp8 = cache->dtype == LI_FP8;
        const int64_t row_bytes =
            fp8 ? cache->r + cache->r / 128 * 4 : (int64_t)cache->r * (cache->dtype == LI_BF16 ? 2 : 4);
        a.stream_nt = stream_nt((int64_t)Q * queries->max_valid * row_bytes);
        if (queries->max_valid > 0) {
            {
                li::TimedScope ts(LI_KERNEL_SCORE_GATHER, stream, true);
                if (fp8)
                    e = li::launch_score_fp8(a, cache->scales, li::fp8_query_scale_offset(Q, H, cache->r), cache->r,
                                             false, queries->max_valid, stream);
                else
                    e = li::launch_score(a, cache->r, cache->dtype == LI_BF16, false, queries->max_valid, stream);
            }
            if (e == hipSuccess && cand_scores) {
                li::TimedScope ts(LI_KERNEL_SELECT, stream);
                e = li::launch_gather_scores(S_pos, M, cand, cand_count, M, cand_scores, Q, stream);
            }
        }
        if (e != hipSuccess) return hip_fail(e, "hs score launch");
        li::SelCall sc{};
        sc.row = li::SelRow{S_pos, M, cand, M, cand, M};
        sc.src_mode = li::kSrcCount;
        sc.cnt = cand_count;
        sc.cnt_cap = M;
        sc.Q = Q;
        sc.k = k;
        sc.max_n = M;
        sc.idx = idx;
        sc.count = count;
        {
            li::TimedScope ts(LI_KERNEL_SELECT, stream);
            e = li::launch_select(sc, sw, false, stream);
        }
        if (e != hipSuccess) return hip_fail(e, "hs select launch");
        return ok();
    }

    li::SelCall sc{};
    sc.row = li::SelRow{S, M, nullptr, 0, cand, M};
    sc.src_mode = li::kSrcCount;
    sc.cnt = cand_count;
    sc.cnt_cap = M;
    sc.Q = Q;
    sc.k = k;
    sc.max_n = M;
    sc.idx = idx;
    sc.count = count;

    hipError_t e = hipSuccess;
    const bool fused_hist = li::selection_wants_counts(Q, M);
    const bool filter_path = fused_hist && li::selection_filters(Q, M); // histogram in the zeroed region
    if (fused_hist && !filter_path) {
        li::TimedScope ts(LI_KERNEL_SELECT, stream);
        e = li::launch_hist_clear(sw, Q, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "histogram clear");
    li::ScoreArgs a = score_args(cache, queries, q_tilde, w, H);
    a.bias = bias;
    a.cand = cand;
    a.cand_count = cand_count;
    a.cand_ld = M;
    a.out = S;
    a.out_ld = M;
    a.max_rows = M;
    a.hist = fused_hist ? sw.hist : nullptr;
    a.flt.filter_path = filter_path;
    {
        li::TimedScope ts(LI_KERNEL_SCORE_GATHER, stream, true);
        if (cache->dtype == LI_FP8)
            e = li::launch_score_fp8(a, cache->scales, li::fp8_query_scale_offset(Q, H, cache->r), cache->r, false, M,
                                     stream);
        else
            e = li::launch_score(a, cache->r, cache->dtype == LI_BF16, false, M, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "hs score launch");
    {
        li::TimedScope ts(LI_KERNEL_SELECT, stream);
        e = li::launch_select(sc, sw, fused_hist, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "hs select launch");
    return ok();
}

size_t li_fp8_query_scale_offset(int32_t Q, int32_t H, int32_t r)
{
    if (Q < 0 || H <= 0 || H > LI_MAX_HEADS || !r_supported(r, LI_FP8)) return 0;
    return (size_t)li::fp8_query_scale_offset(Q, H, r);
}

size_t li_fp8_query_bytes(int32_t Q, int32_t H, int32_t r)
{
    if (Q < 0 || H <= 0 || H > LI_MAX_HEADS || !r_supported(r, LI_FP8)) return 0;
    return (size_t)li::fp8_query_scale_offset(Q, H, r) + (size_t)Q * H * (r / 128) * 4;
}

li_status li_fused_filter(int mode)
{
    if (mode < 0 || mode > 2) return fail(LI_ERR_SHAPE, "fused filter mode %d outside [0, 2]", mode);
    g_fused_filter.store(mode, std::memory_order_relaxed);
    return ok();
}

li_status li_timing_enable(int on)
{
    li::timing_enable(on != 0);
    return ok();
}

li_status li_timing_read(int kernel_class, double *total_ms, int64_t *launches)
{
    if (kernel_class < 0 || kernel_class >= LI_KERNEL_CLASSES)
        return fail(LI_ERR_SHAPE, "kernel class %d outside [0, %d)", kernel_class, (int)LI_KERNEL_CLASSES);
    if (!total_ms || !launches) return fail(LI_ERR_NULL, "total_ms/launches is NULL");
    hipError_t e = li::timing_read(kernel_class, total_ms, launches);
    if (e != hipSuccess) return hip_fail(e, "timing read");
    return ok();
}

li_status li_phase_records(int kernel, void *host, size_t bytes)
{
    if (kernel != LI_PHASE_SCORE_DECODE_BF16 && kernel != LI_PHASE_SCORE_DECODE_FP8)
        return fail(LI_ERR_SHAPE, "phase kernel %d is not LI_PHASE_SCORE_DECODE_BF16/FP8", kernel);
    const size_t full = (size_t)li::kProbeWaves * li::kProbeWords * sizeof(uint64_t);
#ifndef LI_PHASE_PROBE
    (void)host;
    (void)bytes;
    (void)full;
    return fail(LI_ERR_UNSUPPORTED, "phase records exist only in the instrumented (\"phases\") build");
#else
    if (bytes > full) return fail(LI_ERR_SHAPE, "%zu bytes > the %zu bytes of phase records", bytes, full);
    void *dev = nullptr;
    hipError_t e = kernel == LI_PHASE_SCORE_DECODE_BF16 ? li::phase_records_bf16(&dev) : li::phase_records_fp8(&dev);
    if (e != hipSuccess) return hip_fail(e, "phase records address");
    e = host ? hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost) : hipMemset(dev, 0, full);
    if (e != hipSuccess) return hip_fail(e, host ? "phase records copy" : "phase records clear");
    return ok();
#endif
}

} // extern "C"

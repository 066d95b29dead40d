/*
 * latentindex.h — C ABI of the LatentIndex sparse-attention indexer hot path
 * for AMD Instinct MI355X (gfx950).
 *
 * Method: LatentIndex, "Cross-Layer Sharing with Layer-Specific Selection for
 * Sparse Attention" (arXiv:2610.04635), as summarised section by section on
 * paperlayer.ai.  Sections cited below are the paper's.
 *
 *   - A layer group shares one latent cache c_s written by its first (anchor)
 *     layer (§3.1, §B.2).
 *   - Each layer l folds its key decoder into its query,
 *     qt_{l,h} = q_{l,h} W_dec_l (§3.1, §A.2, §B.2), and scores every valid
 *     cached row s as I_l(s) = sum_h w_{l,h} * max(0, qt_{l,h} . c_s).
 *   - Each layer then selects its own top-k rows (§3.1, §4.1: k = 2048).
 *   - Hierarchical selection (HS, §3.2, §C.4): the anchor proposes its top-M
 *     rows (M = 8192 in the paper) and each follower rescores only those and
 *     selects its own top-k within them.
 *   - RoPE-compatible structured decoders (§A.2-§A.4): the latent's rotary
 *     sources are rotated by the native rotary phase before caching, each
 *     layer's per-frequency complex decoder and dense NoPE decoder fold into
 *     its post-RoPE query, and the NoPE output bias becomes one number per
 *     (query, head) added inside the ReLU:
 *     I_l(s) = sum_h w_{l,h} * max(0, qt_{l,h} . c_s + b_{l,h}).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked (host).  Descriptor structs
 *     are host memory read during the call only.
 *   - The caller owns all memory (cache pool, block table, queries, outputs,
 *     workspace).  The library never allocates, frees or synchronizes; every
 *     call only enqueues kernels on `stream` and returns.
 *   - Row-major layouts; int32 indices; `bf16` means IEEE bfloat16 bits.
 *   - Host-side validation happens before anything is enqueued: a failing
 *     call returns a status, enqueues nothing and never aborts.  Values that
 *     live in device memory (sequence ids, seq_lens, block-table entries,
 *     positions, candidates) cannot be checked on the host; the kernels bound
 *     them where they use them (an append whose sequence, position or page
 *     lies outside the cache writes nothing; other indices are clamped into
 *     range), so out-of-range values give meaningless results but never an
 *     access outside the caller's buffers.  NaN/Inf inputs are undefined.
 *   - LI_ERR_HIP reports a failed launch (detail in li_last_error()).
 *   - Calls on different streams are independent; calls that share output
 *     or workspace buffers must be ordered by the caller.
 *   - Three environment variables, read once per process, choose between
 *     equivalent kernels (results are the same within rounding, and up to
 *     the order among equal scores):
 *     LI_DECODE_PATH=lds|vgpr forces the LDS-ring or the register-staged
 *     decode scoring kernel; LI_STREAM_NT=0|1 forces the non-temporal read
 *     policy of the decode latent stream off or on (default: on for
 *     launches that read 128 MiB or more); LI_FUSED_FILTER=0 starts with
 *     the long-row selection's filter pass in a kernel of its own (see
 *     li_fused_filter).
 */
#ifndef LATENTINDEX_H
#define LATENTINDEX_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LI_ABI_VERSION 4
#define LI_API __attribute__((visibility("default")))
#define LI_PAGE_SIZE 64      /* rows per cache page                        */
#define LI_MAX_HEADS 64      /* indexer heads per query                    */
#define LI_MAX_TOPK 65536    /* largest k / M accepted by the selectors    */

typedef enum {
    LI_OK = 0,
    LI_ERR_NULL = 1,        /* a required pointer is NULL                    */
    LI_ERR_SHAPE = 2,       /* a size is non-positive or inconsistent        */
    LI_ERR_UNSUPPORTED = 3, /* valid but not supported (r, H, d, dtype, ...) */
    LI_ERR_WORKSPACE = 4,   /* workspace smaller than li_workspace_bytes()   */
    LI_ERR_HIP = 5          /* a HIP launch failed                           */
} li_status;

/*
 * LI_FP8: segmented FP8 (§B.2: the indexer runs in segmented FP8; §A.2: the
 * decoder is absorbed before the Hadamard rotation).  The pages fix no
 * format; the one implemented: each 128-element segment of a row is rotated
 * by the orthonormal Walsh-Hadamard transform (fp32, butterfly strides 1..64,
 * then x fp32(1/sqrt(128))), given the power-of-two scale 2^e with e the
 * smallest integer such that amax 2^-e <= 448 (clamped to [-120, 120]), and
 * stored as OCP FP8 E4M3 codes of x 2^-e (round to nearest even, saturating
 * at 448).  r must be 128 or 256.
 */
typedef enum { LI_BF16 = 0, LI_FP32 = 1, LI_FP8 = 2 } li_dtype;

/*
 * Shared latent cache of one layer group (§3.1: one cache per group, rows
 * written once by the anchor; §B.2: cached once per group).
 *   pool        [num_pages][page_size][r] of `dtype`; logical row j of
 *               sequence b lives at page block_table[b*max_pages + j/64],
 *               slot j%64.
 *   block_table [batch][max_pages] int32 physical page ids.
 *   seq_lens    [batch] int32 rows present per sequence (after appends).
 *   scales      LI_FP8 only: [num_pages][page_size][r/128] fp32 segment
 *               scales (powers of two) beside the E4M3 codes in pool;
 *               NULL for the other dtypes.
 * page_size must be LI_PAGE_SIZE.  r in {64, 128, 256} for LI_BF16,
 * 1..256 for LI_FP32, {128, 256} for LI_FP8.  A contiguous cache is the
 * identity block table.
 */
typedef struct {
    void *pool;
    const int32_t *block_table;
    const int32_t *seq_lens;
    int32_t batch;
    int32_t max_pages;
    int32_t page_size;
    int32_t num_pages;
    int32_t r;
    li_dtype dtype;
    float *scales;
} li_cache;

/*
 * Queries of one call.  Query i belongs to sequence seq[i] and sits at
 * position pos[i]; it scores rows j < n_i = min(pos[i] + 1, seq_lens[seq[i]])
 * (causal prefix including its own row; §C.4 caps every budget at the valid
 * prefix).  max_valid (host) is an upper bound on every n_i; it sizes the
 * launch grids and the score stride.
 */
typedef struct {
    const int32_t *seq;
    const int32_t *pos;
    int32_t Q;
    int32_t max_valid;
} li_queries;

/*
 * append_latent — the anchor writes T new latent rows into the group cache
 * (§3.1: the shared representation is cached once per group; followers only
 * read it).  rows [T][r] of the cache dtype (bf16 for LI_FP8 caches); row t
 * goes to sequence seq[t], logical position pos[t].  Rows are copied
 * bit-exactly (LI_FP8: rotated and quantized per segment, codes and scale
 * written to the slot).  Updating seq_lens is the caller's job.  Rows that
 * target the same slot race.
 */
LI_API li_status li_append_latent(const li_cache *cache, const void *rows, const int32_t *seq,
                           const int32_t *pos, int32_t T, hipStream_t stream);

/*
 * Rotary layout of a latent row (§A.2, §A.4, §3.1: the RoPE and NoPE
 * branches are concatenated).  The first 2 * sources * freqs elements hold
 * `sources` shared complex sources for each of `freqs` rotary frequencies as
 * (re, im) pairs; pair j is source j / freqs at frequency f = j % freqs.  The
 * rest of the row is the NoPE latent.  The native rotary phase of frequency f
 * at position p is p * theta_f, theta_f = base^(-2f / (2 freqs)) (the RoPE of
 * a native rotary key 2 * freqs wide).
 */
typedef struct {
    int32_t freqs;   /* F >= 1                                       */
    int32_t sources; /* S >= 1; 2 S F <= r                           */
    double base;     /* > 1 (10000 for the usual RoPE)               */
} li_rope;

/*
 * append_latent_rope — li_append_latent for a latent with rotary sources
 * (§A.2: the sources share the native rotary phase, so the latent is rotated
 * before caching).  rows [T][r] hold the unrotated sources (bf16 for LI_BF16
 * and LI_FP8 caches, fp32 for LI_FP32); each source pair of row t is
 * multiplied by exp(i pos[t] theta_f), computed in fp64, and the row is
 * rounded once to the cache dtype (LI_FP8: to fp32, then rotated by the
 * Walsh-Hadamard transform and quantized as li_append_latent does).  The NoPE
 * part is stored as given.  rope (host) as above.
 */
LI_API li_status li_append_latent_rope(const li_cache *cache, const void *rows, const int32_t *seq,
                                const int32_t *pos, int32_t T, const li_rope *rope, hipStream_t stream);

/*
 * absorb_query — qt = q W_dec for every query and head (§3.1, §A.2, §B.2).
 *   q       [Q][H][d]   (dtype)
 *   w_dec   [d][r]      (dtype) the layer's key decoder, latent -> key
 *   q_tilde [Q][H][r]   (dtype) output
 * LI_BF16: bf16 inputs, fp32 accumulation, one round-to-nearest-even to bf16.
 * LI_FP32: fp32 throughout.  H <= 64; r in {64,128,256} and d in
 * {32,64,128,256} for LI_BF16; r in 1..256 and d in 1..1024 for LI_FP32.
 * LI_FP8: bf16 inputs, the products summed in fp64 (exact for bf16 data of
 * ordinary range) and rounded once to fp32, so the result does not depend on
 * the summation order; then each (query, head) segment is rotated and
 * quantized as the cache is (LI_FP8 above); q_tilde is then one
 * buffer of li_fp8_query_bytes(Q, H, r) bytes holding the codes [Q][H][r]
 * followed, at byte offset li_fp8_query_scale_offset(Q, H, r), by the
 * scales [Q][H][r/128] fp32.  r in {128, 256}, d in {32,64,128,256}.
 * LI_FP8 with w_dec NULL (d == r): no decoder; q itself is rotated and
 * quantized (the query of a per-layer indexer scoring its own FP8 keys),
 * exactly as with an identity w_dec.  Other dtypes require w_dec.
 */
LI_API li_status li_absorb_query(const void *q, const void *w_dec, void *q_tilde, int32_t Q, int32_t H,
                          int32_t d, int32_t r, li_dtype dtype, hipStream_t stream);

/*
 * rope_decoder — lowers a layer's structured decoder (§A.4: per-frequency
 * complex coefficients over the shared sources; §A.3: a dense NoPE decoder)
 * into the dense w_dec [d][r] that li_absorb_query takes, so that absorbing a
 * post-RoPE query q = [q_rope (2F, (re, im) pairs) | q_nope (d_nope)] gives
 *   qt[pair (s, f)] = q_f * conj(D[f][s])   and   qt[nope t] = q_nope . Wn[:, t].
 *   D     [F][S][2] (re, im) decoder coefficients, dtype
 *   w_nope [d_nope][r_nope] dtype
 *   w_dec [d][r] out, dtype, d = 2F + d_nope, r = 2SF + r_nope: every entry is
 *         a copy (possibly negated) of a coefficient, or zero, so no rounding
 *         happens here.
 * dtype LI_BF16 or LI_FP32.  rope (host) gives F and S (base is not used).
 */
LI_API li_status li_rope_decoder(const void *D, const void *w_nope, const li_rope *rope, int32_t d_nope,
                          int32_t r_nope, void *w_dec, li_dtype dtype, hipStream_t stream);

/*
 * query_bias — the absorbed NoPE output bias (§A.3: each layer's NoPE
 * decoder carries an output bias beta; k_nope = Wn^T n + beta, so
 * q . k = qt . c + b with b = q_nope . beta, one number per query and head).
 *   q     [Q][H][d] (dtype LI_BF16 or LI_FP32); its last d - d_rope elements
 *         are q_nope
 *   beta  [d - d_rope] fp32
 *   bias  [Q][H] fp32 out: the products summed in fp64 and rounded once.
 */
LI_API li_status li_query_bias(const void *q, const float *beta, int32_t Q, int32_t H, int32_t d, int32_t d_rope,
                        float *bias, li_dtype dtype, hipStream_t stream);

/* Size and scale offset of an LI_FP8 query buffer (0 for invalid sizes). */
LI_API size_t li_fp8_query_bytes(int32_t Q, int32_t H, int32_t r);
LI_API size_t li_fp8_query_scale_offset(int32_t Q, int32_t H, int32_t r);

/*
 * score_topk — full-prefix scoring and per-query top-k (§3.1, §4.1).
 *   q_tilde [Q][H][r] absorbed queries (cache dtype; for an LI_FP8 cache the
 *           FP8 query buffer of li_absorb_query); w [Q][H] fp32 head
 *   weights (any sign); bias [Q][H] fp32 absorbed decoder bias
 *   (li_query_bias) or NULL for none.
 *   scores[i][j] = sum_h w[i][h] max(0, q_tilde[i][h] . c_j + bias[i][h])
 *   for j < n_i, accumulated in fp32.
 *   idx     [Q][k] out: the set of the min(k, n_i) highest-scoring positions
 *           (unordered; slots past count[i] are -1).  Among exactly equal
 *           scores any choice may be returned.
 *   count   [Q]    out: min(k, n_i).
 *   k_inner, idx_inner [Q][k_inner], count_inner [Q]: optional nested
 *           selection (HS anchor, §3.2/§C.4: top-M candidates with the
 *           anchor's own top-k inside them).  k_inner = 0 and NULL pointers
 *           disable it; otherwise 0 < k_inner <= k and idx_inner is a subset
 *           of idx.
 *   scores  [Q][ld] fp32 out (optional, NULL keeps them in the workspace);
 *           ld >= max_valid.  Entries j >= n_i are left untouched.
 *   ws      workspace of at least li_workspace_bytes(op, ...) with op =
 *           LI_OP_SCORE_TOPK (scores == NULL) or LI_OP_SCORE_TOPK_EXT_SCORES.
 * The per-layer baseline indexer (a layer's own key cache of width d, no
 * decoder) is this call on a cache of r = d with q_tilde = q.
 */
LI_API li_status li_score_topk(const li_cache *cache, const li_queries *queries, const void *q_tilde,
                        const float *w, const float *bias, int32_t H, int32_t k, int32_t *idx, int32_t *count,
                        int32_t k_inner, int32_t *idx_inner, int32_t *count_inner, float *scores,
                        int64_t ld, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * score_topk_noalloc — li_score_topk for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments and results without the workspace.
 * The library keeps one scratch array of 32 MiB per GPU (a static device
 * array, held until the process ends) in its place; no call allocates or
 * frees anything.  Calls whose workspace (li_workspace_bytes of
 * LI_OP_SCORE_TOPK, or LI_OP_SCORE_TOPK_EXT_SCORES when scores is given)
 * exceeds 32 MiB return LI_ERR_WORKSPACE without enqueueing anything.  Every
 * call on one GPU shares that GPU's scratch: calls that overlap on one GPU
 * (concurrent streams, threads) race and must be ordered by the caller.
 */
LI_API li_status li_score_topk_noalloc(const li_cache *cache, const li_queries *queries, const void *q_tilde,
                                const float *w, const float *bias, int32_t H, int32_t k, int32_t *idx, int32_t *count,
                                int32_t k_inner, int32_t *idx_inner, int32_t *count_inner, float *scores, int64_t ld,
                                hipStream_t stream);

/*
 * hs_select — HS follower step (§3.2, §3.4, §C.4): rescore only the anchor's
 * candidates with this layer's query and select this layer's top-k of them.
 *   cand       [Q][M] candidate positions (the anchor's idx output with
 *              k = M); cand_count [Q] valid entries per query (<= M).  The
 *              entries must be distinct valid rows of the query's sequence.
 *   idx        [Q][k] out: absolute positions of the min(k, cand_count[i])
 *              best candidates (unordered, -1 padded); count [Q] out.
 *   cand_scores [Q][M] fp32 out (optional): the follower's candidate scores.
 *   ws         at least li_workspace_bytes(LI_OP_HS_SELECT, ...).
 * q_tilde, w and bias as for li_score_topk (the FP8 query buffer for an
 * LI_FP8 cache).
 */
LI_API li_status li_hs_select(const li_cache *cache, const li_queries *queries, const int32_t *cand,
                       const int32_t *cand_count, int32_t M, const void *q_tilde, const float *w,
                       const float *bias, int32_t H, int32_t k, int32_t *idx, int32_t *count, float *cand_scores,
                       void *ws, size_t ws_bytes, hipStream_t stream);

/* Workspace operations:
 *   LI_OP_SCORE_TOPK             li_score_topk with scores == NULL (the score
 *                                rows live in the workspace)
 *   LI_OP_HS_SELECT              li_hs_select
 *   LI_OP_SCORE_TOPK_EXT_SCORES  li_score_topk with a caller score buffer */
enum { LI_OP_SCORE_TOPK = 0, LI_OP_HS_SELECT = 1, LI_OP_SCORE_TOPK_EXT_SCORES = 2 };

/* Workspace bytes for `op` at these sizes (M ignored for the score_topk ops,
 * max_valid ignored for LI_OP_HS_SELECT).  0 means invalid sizes.
 * Every workspace starts with a region of LI_WORKSPACE_ZEROED_BYTES that
 * should be zero before the workspace's first use (e.g. hipMemset once after
 * allocating it): the long-row selection (at most 64 queries over rows
 * longer than 16384) keeps each query's first-digit histogram and counters
 * there instead of clearing them with a kernel of its own, and every call
 * leaves the region zero again.  A region that is not zero costs time, not
 * correctness: the selection finds the histogram inconsistent (its bins do
 * not add up to the row count), selects those queries again from their
 * scores alone (after a wait of up to 1 ms in li_fused_filter mode 1), and
 * leaves the region zero.  The workspaces of li_score_topk and li_hs_select
 * share this layout, so one buffer may serve both (calls in stream order). */
#define LI_WORKSPACE_ZEROED_BYTES (64 * 4112 * 4)
LI_API size_t li_workspace_bytes(int op, int32_t Q, int32_t max_valid, int32_t H, int32_t r, int32_t k,
                          int32_t M);

/*
 * Kernel timing (instrumentation for benchmarks and profiling).  While
 * enabled, the library times each launch of a kernel class with a pair of HIP
 * events on the call's stream.  A scoring class launches one kernel per call,
 * and its events are bound to that kernel's own start and end
 * (hipExtLaunchKernel), as a kernel trace measures it; the other classes
 * record their events on the stream before and after their kernels, so their
 * interval also holds the dispatch of the first kernel after the stream's
 * preceding work (a few microseconds).  li_timing_read waits for the
 * recorded events of one class, returns their summed milliseconds and the
 * number of bracketed launches since the previous read of that class, and
 * forgets them.  Enabling timing creates HIP events (host-side objects; no
 * device memory).  Do not enable it while capturing a HIP graph.
 *   LI_KERNEL_SCORE_DECODE   full-prefix scoring, few queries per sequence
 *   LI_KERNEL_SCORE_PREFILL  full-prefix scoring, many queries per sequence
 *   LI_KERNEL_SCORE_GATHER   HS follower candidate scoring
 *   LI_KERNEL_SELECT         one top-k selection (all of its kernels; in
 *                            li_hs_select also the copy of candidate scores
 *                            when they are asked for)
 *   LI_KERNEL_ABSORB, LI_KERNEL_APPEND
 */
typedef enum {
    LI_KERNEL_SCORE_DECODE = 0,
    LI_KERNEL_SCORE_PREFILL = 1,
    LI_KERNEL_SCORE_GATHER = 2,
    LI_KERNEL_SELECT = 3,
    LI_KERNEL_ABSORB = 4,
    LI_KERNEL_APPEND = 5,
    LI_KERNEL_CLASSES = 6
} li_kernel_class;
LI_API li_status li_timing_enable(int on);
LI_API li_status li_timing_read(int kernel_class, double *total_ms, int64_t *launches);

/*
 * Where the filter pass of a long-row decode selection runs (li_score_topk
 * with at most 64 queries over rows longer than 16384, its first radix
 * digit counted by the scoring kernel).  The pass finds the digit on which
 * the k-th largest score lies and sorts each row into "above" (selected)
 * and "on" (tied, resolved by the final kernel); LatentIndex (paperlayer.ai
 * summary of arXiv:2610.04635), §3.1/§4.1 (per-layer top-k), §3.2 (the HS
 * anchor's nested top-k).
 *   mode 1 (default): inside the decode scoring kernel, when its grid fits
 *          the GPU at once: each workgroup waits (a bounded wait, 1 ms) for
 *          the query's histogram to be complete, then sorts the rows it
 *          holds in LDS.  If the wait runs out (other work held CUs
 *          meanwhile, e.g. another stream's kernels), the final kernel
 *          selects that query again from its scores alone.
 *   mode 0: a kernel of its own after scoring.
 *   mode 2: as 1 with a wait that always runs out at once, so every query
 *          takes the final kernel's fallback (for testing that path).
 * Results are the same in every mode up to the order among equal scores.
 * Process-wide, applies to calls made after it; the initial mode is 1, or
 * 0 when the environment variable LI_FUSED_FILTER=0 is set.  Returns
 * LI_ERR_SHAPE for a mode outside 0..2.
 */
LI_API li_status li_fused_filter(int mode);

/*
 * Phase records of the decode scoring kernels (instrumentation; only the
 * library's "phases" build variant records them, every other build returns
 * LI_ERR_UNSUPPORTED).  In that build each wave of a decode scoring launch
 * writes one record of 8 little-endian uint64 words: five readings of the
 * GPU's 100 MHz constant clock (its start, its first tile of latent rows
 * landed in LDS, the end of its stream, the end of the workgroup barrier
 * after the stream, its end), then (XCC id << 32 | hardware id), blockIdx.x
 * and blockIdx.y.  Record (blockIdx.y * gridDim.x + blockIdx.x) * 4 + wave;
 * 16384 records, zero where no wave wrote.  Each launch overwrites the
 * records its waves write, so read after one launch.
 * li_phase_records(kernel, host, bytes): host != NULL copies the first
 * `bytes` bytes (at most 16384 * 64) of that kernel's records on the current
 * device to host memory (synchronous); host == NULL zeroes them.
 */
typedef enum { LI_PHASE_SCORE_DECODE_BF16 = 0, LI_PHASE_SCORE_DECODE_FP8 = 1 } li_phase_kernel;
LI_API li_status li_phase_records(int kernel, void *host, size_t bytes);

LI_API const char *li_status_str(li_status s);
/* Detail of the last failure on the calling thread ("" if none). */
LI_API const char *li_last_error(void);
LI_API int32_t li_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LATENTINDEX_H */

// Host-side driver of the C ABI for the AddressSanitizer build: every entry
// point is called through its validation paths (NULL descriptors and
// pointers, inconsistent sizes, unsupported shapes, a short workspace), each
// of which must return its status without enqueueing work, so no GPU is
// needed.  ASan checks the host code on the way (error formatting, the
// thread-local error string, the size arithmetic).  Exit status 0 = every
// expectation held.
#include <stdio.h>
#include <string.h>

#include "latentindex.h"

static int failures = 0;

static void expect(li_status got, li_status want, const char *what)
{
    if (got != want) {
        printf("FAIL %s: %s (want %s): %s\n", what, li_status_str(got), li_status_str(want), li_last_error());
        ++failures;
    } else if (got != LI_OK && strlen(li_last_error()) == 0) {
        printf("FAIL %s: no error detail\n", what);
        ++failures;
    }
}

int main()
{
    void *const FAKE = (void *)0x10000; // never dereferenced: validation fails first
    int32_t *const IFAKE = (int32_t *)FAKE;
    float *const FFAKE = (float *)FAKE;
    if (li_abi_version() != LI_ABI_VERSION) {
        printf("FAIL abi version\n");
        return 1;
    }
    for (int s = 0; s <= 6; ++s) (void)strlen(li_status_str((li_status)s));

    li_cache c;
    memset(&c, 0, sizeof c);
    c.pool = FAKE;
    c.block_table = IFAKE;
    c.seq_lens = IFAKE;
    c.batch = 2;
    c.max_pages = 4;
    c.page_size = LI_PAGE_SIZE;
    c.num_pages = 8;
    c.r = 256;
    c.dtype = LI_BF16;
    li_queries q;
    memset(&q, 0, sizeof q);
    q.seq = IFAKE;
    q.pos = IFAKE;
    q.Q = 2;
    q.max_valid = 200;

    // append
    expect(li_append_latent(nullptr, FAKE, IFAKE, IFAKE, 1, nullptr), LI_ERR_NULL, "append NULL cache");
    expect(li_append_latent(&c, nullptr, IFAKE, IFAKE, 1, nullptr), LI_ERR_NULL, "append NULL rows");
    expect(li_append_latent(&c, FAKE, IFAKE, IFAKE, -1, nullptr), LI_ERR_SHAPE, "append T<0");
    expect(li_append_latent(&c, FAKE, IFAKE, IFAKE, 0, nullptr), LI_OK, "append T=0");
    li_cache bad = c;
    bad.page_size = 32;
    expect(li_append_latent(&bad, FAKE, IFAKE, IFAKE, 1, nullptr), LI_ERR_UNSUPPORTED, "append page size");
    bad = c;
    bad.r = 96;
    expect(li_append_latent(&bad, FAKE, IFAKE, IFAKE, 1, nullptr), LI_ERR_UNSUPPORTED, "append r");
    bad = c;
    bad.dtype = LI_FP8;
    expect(li_append_latent(&bad, FAKE, IFAKE, IFAKE, 1, nullptr), LI_ERR_NULL, "append FP8 without scales");
    li_rope rope = {64, 4, 10000.0};
    expect(li_append_latent_rope(&c, FAKE, IFAKE, IFAKE, 1, &rope, nullptr), LI_ERR_SHAPE, "rope 2SF > r");
    rope = {16, 2, 0.5};
    expect(li_append_latent_rope(&c, FAKE, IFAKE, IFAKE, 1, &rope, nullptr), LI_ERR_SHAPE, "rope base");
    expect(li_append_latent_rope(&c, FAKE, IFAKE, IFAKE, 1, nullptr, nullptr), LI_ERR_NULL, "rope NULL");

    // absorb, decoder lowering, bias
    expect(li_absorb_query(FAKE, FAKE, FAKE, 1, 65, 128, 256, LI_BF16, nullptr), LI_ERR_SHAPE, "absorb H");
    expect(li_absorb_query(FAKE, FAKE, FAKE, 1, 64, 100, 256, LI_BF16, nullptr), LI_ERR_UNSUPPORTED, "absorb d");
    expect(li_absorb_query(FAKE, nullptr, FAKE, 1, 64, 128, 256, LI_BF16, nullptr), LI_ERR_NULL, "absorb no W");
    expect(li_absorb_query(FAKE, nullptr, FAKE, 1, 64, 128, 256, LI_FP8, nullptr), LI_ERR_SHAPE, "absorb FP8 d!=r");
    expect(li_absorb_query(FAKE, FAKE, FAKE, 0, 64, 128, 256, LI_BF16, nullptr), LI_OK, "absorb Q=0");
    rope = {16, 2, 10000.0};
    expect(li_rope_decoder(FAKE, FAKE, &rope, -1, 4, FAKE, LI_BF16, nullptr), LI_ERR_SHAPE, "decoder d_nope");
    expect(li_rope_decoder(FAKE, FAKE, &rope, 4, 4, FAKE, LI_FP8, nullptr), LI_ERR_UNSUPPORTED, "decoder dtype");
    expect(li_query_bias(FAKE, FFAKE, 1, 4, 8, 9, FFAKE, LI_BF16, nullptr), LI_ERR_SHAPE, "bias d_rope > d");

    // score + top-k
    const size_t ws = li_workspace_bytes(LI_OP_SCORE_TOPK, 2, 200, 64, 256, 64, 0);
    if (ws == 0 || li_workspace_bytes(LI_OP_SCORE_TOPK, 2, 200, 64, 256, 0, 0) != 0) {
        printf("FAIL workspace sizes\n");
        ++failures;
    }
    expect(li_score_topk(&c, &q, FAKE, FFAKE, nullptr, 64, 64, IFAKE, IFAKE, 0, nullptr, nullptr, nullptr, 0, FAKE,
                         ws - 1, nullptr),
           LI_ERR_WORKSPACE, "score_topk short workspace");
    expect(li_score_topk(&c, &q, FAKE, FFAKE, nullptr, 64, 64, IFAKE, IFAKE, 65, IFAKE, IFAKE, nullptr, 0, FAKE, ws,
                         nullptr),
           LI_ERR_SHAPE, "score_topk k_inner > k");
    expect(li_score_topk(&c, &q, FAKE, FFAKE, nullptr, 64, 64, IFAKE, IFAKE, 8, nullptr, IFAKE, nullptr, 0, FAKE, ws,
                         nullptr),
           LI_ERR_NULL, "score_topk inner NULL");
    expect(li_score_topk(&c, &q, FAKE, FFAKE, nullptr, 64, 64, IFAKE, IFAKE, 0, nullptr, nullptr, FFAKE, 199, FAKE,
                         ws, nullptr),
           LI_ERR_SHAPE, "score_topk ld < max_valid");
    li_queries bq = q;
    bq.max_valid = 4 * 64 + 1;
    expect(li_score_topk(&c, &bq, FAKE, FFAKE, nullptr, 64, 64, IFAKE, IFAKE, 0, nullptr, nullptr, nullptr, 0, FAKE,
                         ws, nullptr),
           LI_ERR_SHAPE, "score_topk max_valid > capacity");
    expect(li_score_topk_noalloc(&c, &q, FAKE, FFAKE, nullptr, 64, 0, IFAKE, IFAKE, 0, nullptr, nullptr, nullptr, 0,
                                 nullptr),
           LI_ERR_SHAPE, "noalloc k=0");
    li_queries big = q;
    big.Q = 2000;
    big.max_valid = 256;
    li_cache bigc = c;
    bigc.max_pages = 65536 / 64;
    big.max_valid = 65536;
    expect(li_score_topk_noalloc(&bigc, &big, FAKE, FFAKE, nullptr, 64, 64, IFAKE, IFAKE, 0, nullptr, nullptr,
                                 nullptr, 0, nullptr),
           LI_ERR_WORKSPACE, "noalloc beyond its scratch");

    // follower select
    const size_t wh = li_workspace_bytes(LI_OP_HS_SELECT, 2, 0, 64, 256, 64, 512);
    expect(li_hs_select(&c, &q, IFAKE, IFAKE, 512, FAKE, FFAKE, nullptr, 64, 64, IFAKE, IFAKE, nullptr, FAKE, wh - 1,
                        nullptr),
           LI_ERR_WORKSPACE, "hs_select short workspace");
    expect(li_hs_select(&c, &q, nullptr, IFAKE, 512, FAKE, FFAKE, nullptr, 64, 64, IFAKE, IFAKE, nullptr, FAKE, wh,
                        nullptr),
           LI_ERR_NULL, "hs_select NULL cand");
    expect(li_hs_select(&c, &q, IFAKE, IFAKE, 0, FAKE, FFAKE, nullptr, 64, 64, IFAKE, IFAKE, nullptr, FAKE, wh,
                        nullptr),
           LI_ERR_SHAPE, "hs_select M=0");

    // sizes and timing classes
    if (li_fp8_query_bytes(1, 64, 256) == 0 || li_fp8_query_bytes(1, 64, 96) != 0) {
        printf("FAIL fp8 query bytes\n");
        ++failures;
    }
    double ms = 0.0;
    int64_t n = 0;
    expect(li_timing_read(99, &ms, &n), LI_ERR_SHAPE, "timing class");
    expect(li_timing_read(0, nullptr, &n), LI_ERR_NULL, "timing NULL");
    expect(li_fused_filter(3), LI_ERR_SHAPE, "fused filter mode");
    expect(li_fused_filter(1), LI_OK, "fused filter mode 1");
    printf("%s: %d failures\n", failures ? "FAIL" : "ok", failures);
    return failures ? 1 : 0;
}

/*
 * LatentIndex indexer: plain CPU oracle (fp64).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or constant with the GPU library and is written to be read against
 * the LatentIndex paper (paperlayer.ai section-by-section summary of
 * arXiv:2610.04635, "LatentIndex: Cross-Layer Sharing with Layer-Specific
 * Selection for Sparse Attention"), cited below by section.
 *
 * Every input is an fp64 copy of the exact stored values; every sum is a
 * plain loop in fp64 with no blocking, fusion or reordering.  Paging never
 * enters here: the latent of one sequence is a contiguous [n][r] array.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/*
 * Query-side decoder absorption (§3.1 and §A.2/§B.2: each layer folds its
 * key decoder into its query so that it scores the shared latent directly).
 *   qt[i][h][t] = sum_e q[i][h][e] * W[e][t]
 * q: [Q][H][d]   W: [d][r] (the layer's decoder, latent -> key)   qt: [Q][H][r]
 */
void lio_absorb(const double *q, const double *W, int64_t Q, int64_t H, int64_t d, int64_t r,
                double *qt)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < Q * H; ++i) {
        const double *qi = q + i * d;
        double *out = qt + i * r;
        for (int64_t t = 0; t < r; ++t) {
            double acc = 0.0;
            for (int64_t e = 0; e < d; ++e)
                acc += qi[e] * W[e * r + t];
            out[t] = acc;
        }
    }
}

/*
 * Layer-specific scoring of latent rows (§3.1, §B.2: the layer keeps its own
 * query and head weights and scores the shared cache):
 *   s[i] = sum_h w[h] * max(0, sum_t qt[h][t] * C[row_i][t])
 * where row_i = rows[i] when rows != NULL, else row_i = i.
 * qt: [H][r] one absorbed query   w: [H]   C: latent [*][r]   s: [m]
 */
void lio_score(const double *qt, const double *w, const double *C, const int32_t *rows, int64_t m,
               int64_t H, int64_t r, double *s)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i) {
        const int64_t row = rows ? (int64_t)rows[i] : i;
        const double *c = C + row * r;
        double total = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            double dot = 0.0;
            for (int64_t t = 0; t < r; ++t)
                dot += qt[h * r + t] * c[t];
            total += w[h] * (dot > 0.0 ? dot : 0.0);
        }
        s[i] = total;
    }
}

/*
 * The same score computed the long way, by rebuilding each row's effective
 * key first (what absorption avoids, §3.1; the per-layer key cache of the
 * native indexer, §1):
 *   K[j][e] = sum_t W[e][t] * C[j][t]            (the layer's key for row j)
 *   s[j]    = sum_h w[h] * max(0, sum_e q[h][e] * K[j][e])
 * q: [H][d] un-absorbed query   W: [d][r]   C: [n][r]   s: [n]
 * Called with W = NULL it scores C as explicit keys (r must equal d): the
 * per-layer baseline indexer on its own key cache.
 */
void lio_score_explicit(const double *q, const double *W, const double *w, const double *C,
                        int64_t n, int64_t H, int64_t d, int64_t r, double *s)
{
#pragma omp parallel
    {
        double *key = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(static)
        for (int64_t j = 0; j < n; ++j) {
            const double *c = C + j * r;
            for (int64_t e = 0; e < d; ++e) {
                if (W) {
                    double acc = 0.0;
                    for (int64_t t = 0; t < r; ++t)
                        acc += W[e * r + t] * c[t];
                    key[e] = acc;
                } else {
                    key[e] = c[e];
                }
            }
            double total = 0.0;
            for (int64_t h = 0; h < H; ++h) {
                double dot = 0.0;
                for (int64_t e = 0; e < d; ++e)
                    dot += q[h * d + e] * key[e];
                total += w[h] * (dot > 0.0 ? dot : 0.0);
            }
            s[j] = total;
        }
        free(key);
    }
}

/*
 * Top-K selection (§3.1: every layer selects its own tokens; §4.1: up to
 * 2048 per query; §C.4: budgets are capped by the valid prefix).
 * The m entries are (score s[i], position pos[i]) (pos == NULL means
 * pos[i] = i).  They are ordered by score descending, then position
 * ascending, with a full sort; out receives the positions of the first K.
 * Returns K, or -1 on allocation failure.
 */
typedef struct {
    double s;
    int32_t p;
} lio_entry;

static int lio_cmp(const void *a, const void *b)
{
    const lio_entry *x = (const lio_entry *)a, *y = (const lio_entry *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->p > y->p) - (x->p < y->p);
}

int64_t lio_topk(const double *s, const int32_t *pos, int64_t m, int64_t K, int32_t *out)
{
    if (K > m) K = m;
    if (K <= 0) return 0;
    lio_entry *e = (lio_entry *)malloc(sizeof(lio_entry) * (size_t)m);
    if (!e) return -1;
    for (int64_t i = 0; i < m; ++i) {
        e[i].s = s[i];
        e[i].p = pos ? pos[i] : (int32_t)i;
    }
    qsort(e, (size_t)m, sizeof(lio_entry), lio_cmp);
    for (int64_t i = 0; i < K; ++i)
        out[i] = e[i].p;
    free(e);
    return K;
}

/* Number of threads the OpenMP loops above run with in this process. */
int lio_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

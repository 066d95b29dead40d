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
 *   s[i] = sum_h w[h] * max(0, sum_t qt[h][t] * C[row_i][t] + b[h])
 * where row_i = rows[i] when rows != NULL, else row_i = i, and b[h] is the
 * absorbed decoder bias (§A.3: each layer's NoPE decoder carries an output
 * bias; its dot with the query is one number per head), 0 when bias == NULL.
 * qt: [H][r] one absorbed query   w: [H]   bias: [H] or NULL
 * C: latent [*][r]   s: [m]
 */
void lio_score(const double *qt, const double *w, const double *bias, const double *C, const int32_t *rows,
               int64_t m, int64_t H, int64_t r, double *s)
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
            if (bias) dot += bias[h];
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

/*
 * Segmented FP8 storage and scoring (§B.2: the indexer runs in segmented
 * FP8; §A.2: queries are absorbed before the Hadamard rotation, i.e. the
 * rotation is applied to both sides ahead of quantization).  The pages give
 * neither formats nor segment sizes; the reading implemented here:
 *   - each 128-element segment of a row is rotated by the orthonormal
 *     Walsh-Hadamard transform (fp32 butterflies, strides 1, 2, ..., 64,
 *     then a multiply by the fp32 value of 1/sqrt(128));
 *   - the segment gets a power-of-two scale 2^e, e the smallest integer
 *     with amax * 2^-e <= 448 (clamped to [-120, 120]);
 *   - every element becomes an OCP FP8 E4M3 code of x * 2^-e, rounded to
 *     nearest-even and saturated at 448.
 * Rotation is orthonormal, so the score of the rotated, unquantized rows
 * equals the plain score; quantization is the only approximation.
 */

/* Value of an OCP E4M3 code: 1 sign, 4 exponent (bias 7), 3 mantissa bits. */
double lio_e4m3_decode(uint8_t c)
{
    const int ex = (c >> 3) & 15, m = c & 7;
    const double v = ex == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), ex - 10);
    return (c & 0x80) ? -v : v;
}

/* Nearest E4M3 code (ties to even mantissa); magnitudes of 448 and above
 * become 448.  v must not be NaN. */
uint8_t lio_e4m3_encode(float v)
{
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    const float a = fabsf(v);
    if (!(a > 0.0f)) return sign;
    if (a >= 448.0f) return sign | 0x7E;
    int E;
    frexpf(a, &E);           /* a = f 2^E, f in [0.5, 1) */
    const int e = E - 1;     /* floor(log2 a) */
    if (e < -6) {            /* below the smallest normal: steps of 2^-9 */
        const float n = rintf(ldexpf(a, 9));
        return sign | (uint8_t)n;      /* n = 8 is the smallest normal, code 8 */
    }
    int m = (int)rintf(ldexpf(a, 3 - e)); /* 8 .. 16 */
    int ee = e;
    if (m == 16) {
        m = 8;
        ee += 1;
    }
    return sign | (uint8_t)(((ee + 7) << 3) | (m - 8));
}

/* In-place orthonormal Walsh-Hadamard transform of 128 floats (fp32). */
void lio_wht128(float *x)
{
    for (int h = 1; h < 128; h <<= 1)
        for (int i = 0; i < 128; i += 2 * h)
            for (int j = i; j < i + h; ++j) {
                const float a = x[j], b = x[j + h];
                x[j] = a + b;
                x[j + h] = a - b;
            }
    const float k = 0.08838834764831845f; /* 1/sqrt(128) */
    for (int j = 0; j < 128; ++j)
        x[j] = x[j] * k;
}

/* Smallest e with amax * 2^-e <= 448 (0 for amax == 0), clamped. */
int lio_pow2_exponent(float amax)
{
    if (!(amax > 0.0f)) return 0;
    int E;
    const float f = frexpf(amax, &E); /* amax = (2f) 2^(E-1), 2f in [1, 2) */
    int e = (2.0f * f <= 1.75f) ? E - 9 : E - 8;
    if (e < -120) e = -120;
    if (e > 120) e = 120;
    return e;
}

/* Rows [rows][r] (r a multiple of 128) -> codes [rows][r] and one scale
 * per (row, segment), [rows][r/128]. */
void lio_quantize_rows(const float *x, int64_t rows, int64_t r, uint8_t *codes, float *scales)
{
    const int64_t nseg = r / 128;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        for (int64_t g = 0; g < nseg; ++g) {
            float y[128];
            for (int t = 0; t < 128; ++t)
                y[t] = x[i * r + g * 128 + t];
            lio_wht128(y);
            float amax = 0.0f;
            for (int t = 0; t < 128; ++t)
                amax = fmaxf(amax, fabsf(y[t]));
            const int e = lio_pow2_exponent(amax);
            scales[i * nseg + g] = ldexpf(1.0f, e);
            for (int t = 0; t < 128; ++t)
                codes[i * r + g * 128 + t] = lio_e4m3_encode(ldexpf(y[t], -e));
        }
    }
}

/*
 * Score from FP8 rows (§3.1 score on the rotated, quantized operands):
 *   s[i] = sum_h w[h] max(0, sum_g qs[h][g] cs[row_i][g]
 *                                 sum_{t in segment g} dec(qc[h][t]) dec(cc[row_i][t])
 *                            + b[h])      (b: the absorbed decoder bias, or 0)
 * qc: [H][r] codes, qs: [H][r/128]; cc: [*][r] codes, cs: [*][r/128];
 * row_i = rows[i] when rows != NULL, else i.
 */
void lio_score_fp8(const uint8_t *qc, const float *qs, const double *w, const double *bias, const uint8_t *cc,
                   const float *cs, const int32_t *rows, int64_t m, int64_t H, int64_t r, double *s)
{
    const int64_t nseg = r / 128;
    /* the value of every code, as lio_e4m3_decode gives it, looked up instead
     * of recomputed per product (the same values in the same order) */
    double dec[256];
    for (int c = 0; c < 256; ++c)
        dec[c] = lio_e4m3_decode((uint8_t)c);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i) {
        const int64_t row = rows ? (int64_t)rows[i] : i;
        double total = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            double dot = 0.0;
            for (int64_t g = 0; g < nseg; ++g) {
                double seg = 0.0;
                for (int t = 0; t < 128; ++t)
                    seg += dec[qc[h * r + g * 128 + t]] * dec[cc[row * r + g * 128 + t]];
                dot += (double)qs[h * nseg + g] * (double)cs[row * nseg + g] * seg;
            }
            if (bias) dot += bias[h];
            total += w[h] * (dot > 0.0 ? dot : 0.0);
        }
        s[i] = total;
    }
}

/*
 * RoPE-compatible structured decoder (§A.2, §A.4, §A.3; §3.1: one latent
 * row holds the rotary part followed by the NoPE part, and the group keeps
 * a single copy of it).
 *
 * Latent row layout: the first 2*S*F elements are S shared complex sources
 * for each of F rotary frequencies, stored as (re, im) pairs; pair j holds
 * source s = j / F at frequency f = j % F.  The remaining r_nope elements are
 * the NoPE latent.  The native indexer key of a layer is
 * [k_rope (2F: F complex, (re, im) pairs) | k_nope (d_nope)].
 *
 * Rotary phase of frequency f at position p: p * theta_f with
 * theta_f = base^(-2f / (2F)), the native RoPE of a 2F-wide rotary key.
 */
static double lio_theta(int64_t f, int64_t F, double base)
{
    return pow(base, -(double)(2 * f) / (double)(2 * F));
}

/*
 * The sources share the native rotary phase, so the cached latent is rotated
 * before caching (§A.2): each source pair of row i is multiplied by
 * exp(i * pos[i] * theta_f).  rows: [n][r], in place; the NoPE part is left
 * as it is.
 */
void lio_rope_rotate(double *rows, const int32_t *pos, int64_t n, int64_t r, int64_t F, int64_t S, double base)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double *x = rows + i * r;
        for (int64_t j = 0; j < S * F; ++j) {
            const int64_t f = j % F;
            const double ang = (double)pos[i] * lio_theta(f, F, base);
            const double c = cos(ang), sn = sin(ang);
            const double re = x[2 * j], im = x[2 * j + 1];
            x[2 * j] = re * c - im * sn;
            x[2 * j + 1] = re * sn + im * c;
        }
    }
}

/*
 * Absorption of the structured decoder into a post-RoPE query (§A.2: the
 * decoder is absorbed into post-RoPE queries; §A.4: per frequency, layer
 * decoder coefficients D[f][s] over shared complex sources; §A.3: a dense
 * NoPE decoder Wn and an output bias beta).
 *   rope slot (s, f):  qt = q_f * conj(D[f][s])     (q_f = q[2f] + i q[2f+1])
 *   NoPE column t:     qt = sum_e q[2F + e] * Wn[e][t]
 *   bias:              b  = sum_e q[2F + e] * beta[e]
 * q: [QH][2F + d_nope]; D: [F][S][2] (re, im); Wn: [d_nope][r_nope];
 * beta: [d_nope]; qt: [QH][2SF + r_nope]; b: [QH].
 */
void lio_absorb_rope(const double *q, const double *D, const double *Wn, const double *beta, int64_t QH,
                     int64_t F, int64_t S, int64_t d_nope, int64_t r_nope, double *qt, double *b)
{
    const int64_t d = 2 * F + d_nope, r = 2 * S * F + r_nope;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < QH; ++i) {
        const double *qi = q + i * d;
        double *out = qt + i * r;
        for (int64_t s = 0; s < S; ++s)
            for (int64_t f = 0; f < F; ++f) {
                const double a = qi[2 * f], bb = qi[2 * f + 1];
                const double c = D[(f * S + s) * 2], e = D[(f * S + s) * 2 + 1];
                /* (a + i bb)(c - i e) */
                out[2 * (s * F + f)] = a * c + bb * e;
                out[2 * (s * F + f) + 1] = bb * c - a * e;
            }
        for (int64_t t = 0; t < r_nope; ++t) {
            double acc = 0.0;
            for (int64_t e = 0; e < d_nope; ++e)
                acc += qi[2 * F + e] * Wn[e * r_nope + t];
            out[2 * S * F + t] = acc;
        }
        double acc = 0.0;
        for (int64_t e = 0; e < d_nope; ++e)
            acc += qi[2 * F + e] * beta[e];
        b[i] = acc;
    }
}

/*
 * The same score the long way (§3.1, §A.2): rebuild each row's native key
 * from the unrotated latent, apply the native RoPE at the row's position to
 * the decoded rotary key, and score with the un-absorbed post-RoPE query:
 *   k_f    = exp(i pos theta_f) * sum_s D[f][s] z_{s,f}
 *   k_nope = Wn^T n + beta
 *   s[j]   = sum_h w[h] max(0, q_h . [k_rope | k_nope])
 * q: [H][2F + d_nope]; C: unrotated latent rows [n][2SF + r_nope]; pos: [n].
 */
void lio_score_explicit_rope(const double *q, const double *D, const double *Wn, const double *beta, const double *w,
                             const double *C, const int32_t *pos, int64_t n, int64_t H, int64_t F, int64_t S,
                             int64_t d_nope, int64_t r_nope, double base, double *s)
{
    const int64_t d = 2 * F + d_nope, r = 2 * S * F + r_nope;
#pragma omp parallel
    {
        double *key = (double *)malloc(sizeof(double) * (size_t)(d > 0 ? d : 1));
#pragma omp for schedule(static)
        for (int64_t j = 0; j < n; ++j) {
            const double *c = C + j * r;
            for (int64_t f = 0; f < F; ++f) {
                double kr = 0.0, ki = 0.0;
                for (int64_t src = 0; src < S; ++src) {
                    const double dr = D[(f * S + src) * 2], di = D[(f * S + src) * 2 + 1];
                    const double zr = c[2 * (src * F + f)], zi = c[2 * (src * F + f) + 1];
                    kr += dr * zr - di * zi;
                    ki += dr * zi + di * zr;
                }
                const double ang = (double)pos[j] * lio_theta(f, F, base);
                key[2 * f] = kr * cos(ang) - ki * sin(ang);
                key[2 * f + 1] = kr * sin(ang) + ki * cos(ang);
            }
            for (int64_t e = 0; e < d_nope; ++e) {
                double acc = beta[e];
                for (int64_t t = 0; t < r_nope; ++t)
                    acc += Wn[e * r_nope + t] * c[2 * S * F + t];
                key[2 * F + e] = acc;
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

/* Number of threads the OpenMP loops above run with in this process. */
int lio_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Plain CPU oracle for decode attention over a shared-head KV cache.
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, bench CPU baseline); never
 * linked into or called by the product path. See oracle.h for the sources.
 *
 * Every floating-point sum here is a plain left-to-right loop in double.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* fp8 e4m3 (OCP "E4M3FN"): sign, 4 exponent bits (bias 7), 3 mantissa bits;
 * exponent 0 holds the subnormals m/8 * 2^-6; S.1111.111 is NaN and there is
 * no infinity, so the largest finite value is 1.75 * 2^8 = 448. */
double oracle_fp8_e4m3_decode(uint8_t c) {
    int e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double v = e == 0 ? (m / 8.0) * ldexp(1.0, -6) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
    return (c & 0x80) ? -v : v;
}

/* Nearest e4m3 value, ties to the even code; magnitudes at or above 448
 * saturate to +-448 (a finite input never becomes NaN); NaN stays NaN. */
uint8_t oracle_fp8_e4m3_encode(float f) {
    uint8_t sign = signbit(f) ? 0x80 : 0;
    float a = fabsf(f);
    if (isnan(f)) return sign | 0x7F;
    if (a >= 448.0f) return sign | 0x7E;
    if (a < 0.015625f) /* below 2^-6: the multiples of 2^-9 (8 * 2^-9 is 2^-6, code 8) */
        return sign | (uint8_t)nearbyintf(a * 512.0f);
    int e;
    float fr = frexpf(a, &e);             /* a = fr * 2^e, fr in [0.5, 1) */
    int sm = (int)nearbyintf(fr * 16.0f); /* 8 + mantissa, rounded: 8 .. 16 */
    int E = e - 1 + 7;                    /* biased exponent of 2^(e-1) */
    if (sm == 16) {
        sm = 8;
        E += 1;
    }
    return sign | (uint8_t)((E << 3) | (sm - 8));
}

/* int8 codes, two's complement: the code itself is the value before the
 * head's scale. Encoding: nearest integer, ties to even (the default
 * rounding mode), saturating at +-127 (-128 is never produced, so the codes
 * are symmetric about 0); NaN becomes 0. */
double oracle_int8_decode(int8_t c) { return (double)c; }

int8_t oracle_int8_encode(float f) {
    if (isnan(f)) return 0;
    float r = nearbyintf(f);
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    return (int8_t)r;
}

/* Read element idx of a buffer of the given type, widened exactly to double. */
static double elem(const void *base, size_t idx, int dtype) {
    if (dtype == ORACLE_FP8_E4M3) return oracle_fp8_e4m3_decode(((const uint8_t *)base)[idx]);
    if (dtype == ORACLE_INT8) return oracle_int8_decode(((const int8_t *)base)[idx]);
    if (dtype == ORACLE_F32) {
        float f;
        memcpy(&f, (const char *)base + 4 * idx, 4);
        return (double)f;
    }
    uint16_t hbits;
    memcpy(&hbits, (const char *)base + 2 * idx, 2);
    uint32_t u = (uint32_t)hbits << 16; /* bfloat16 = top half of binary32 */
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static size_t elem_bytes(int dtype) {
    return dtype == ORACLE_F32 ? 4u : (dtype == ORACLE_FP8_E4M3 || dtype == ORACLE_INT8) ? 1u : 2u;
}

int oracle_append_kv_multi(void *k_cache, void *v_cache, const void *k_new,
                           const void *v_new, const int32_t *seq_lens, int b,
                           int T, int g, int S, int d, int dtype) {
    if (b < 1 || T < 1 || g < 1 || S < 1 || d < 1) return ORACLE_BAD_SHAPE;
    int rc = ORACLE_OK;
    size_t eb = elem_bytes(dtype);
    size_t row = (size_t)d * eb;
    for (int i = 0; i < b; i++) {
        int L = seq_lens[i];
        if (L < T || L > S) { /* never truncate or wrap silently */
            rc |= ORACLE_BAD_LEN;
            continue;
        }
        /* token tau of this step is position L - T + tau */
        for (int tau = 0; tau < T; tau++)
            for (int j = 0; j < g; j++) {
                size_t dst = (((size_t)i * g + j) * S + (size_t)(L - T + tau)) * row;
                size_t src = (((size_t)i * T + tau) * g + j) * row;
                memcpy((char *)k_cache + dst, (const char *)k_new + src, row);
                memcpy((char *)v_cache + dst, (const char *)v_new + src, row);
            }
    }
    return rc;
}

int oracle_append_kv(void *k_cache, void *v_cache, const void *k_new,
                     const void *v_new, const int32_t *seq_lens, int b, int g,
                     int S, int d, int dtype) {
    return oracle_append_kv_multi(k_cache, v_cache, k_new, v_new, seq_lens, b, 1,
                                  g, S, d, dtype);
}

/* ---- decode attention: one (sequence, query head) row ---------------- */

typedef struct {
    const void *q, *k, *v;
    const int32_t *seq_lens;
    int b, T, h, g, S, d, dtype; /* T query tokens per sequence; dtype: K and V */
    double scale;
    double *out, *alpha;
    int row_begin, row_end; /* rows are (i*T + tau)*h + hq */
    int flags;
    /* paged cache (block_table != NULL): position t of sequence i is row
     * t % page_size of page block_table[i * max_pages + t / page_size] */
    const int32_t *block_table;
    int page_size, max_pages, num_pages;
    /* element type of q; per-K/V-head dequantisation scales of a quantised
     * cache (NULL: none): a cache value is code * scale[j] */
    int q_dtype;
    const float *k_scale, *v_scale;
    int window; /* > 0: a query at position p sees only t > p - window */
} decode_job;

/* Element index of K/V row (sequence i, K/V head j, position t), or -1 when
 * the page holding it is not a valid page id. */
static long long kv_row(const decode_job *J, int i, int j, int t) {
    if (!J->block_table) return (((long long)i * J->g + j) * J->S + t) * J->d;
    int page = J->block_table[(size_t)i * J->max_pages + t / J->page_size];
    if (page < 0 || page >= J->num_pages) return -1;
    return (((long long)page * J->g + j) * J->page_size + t % J->page_size) * J->d;
}

static void decode_row(decode_job *J, int row) {
    int hq = row % J->h, it = row / J->h;
    int i = it / J->T, tau = it % J->T;
    int d = J->d, S = J->S;
    int G = J->h / J->g;      /* query heads per K/V head */
    int j = hq / G;           /* [GQA notes] §五: j = i // (h/g) */
    int L = J->seq_lens[i];
    double *o = J->out + (size_t)row * d;
    if (L < J->T || L > S) {
        for (int x = 0; x < d; x++) o[x] = NAN;
        J->flags |= ORACLE_BAD_LEN;
        return;
    }
    /* The step's T tokens are positions L-T .. L-1; token tau sees the
     * positions up to its own, t <= L-T+tau (the causal mask is applied per
     * query position, shared K/V or not: [GQA notes] §十 item 10). */
    int A = L - J->T + 1 + tau;
    /* a sliding window of W positions keeps t in [A - W, A) (the window
     * start replaces 0; the GQA + SWA models of [MQA concept] 玩家對比) */
    int a0 = (J->window > 0 && A > J->window) ? A - J->window : 0;
    size_t qoff = (size_t)row * d;
    for (int t = a0; t < A; t++) {
        if (kv_row(J, i, j, t) < 0) { /* a position on an invalid page */
            for (int x = 0; x < d; x++) o[x] = NAN;
            J->flags |= ORACLE_BAD_PAGE;
            return;
        }
    }

    double ks = J->k_scale ? (double)J->k_scale[j] : 1.0;
    double vs = J->v_scale ? (double)J->v_scale[j] : 1.0;
    double *s = (double *)malloc(sizeof(double) * (size_t)A);
    /* score_t = (Q_i . K_j,t) * scale */
    for (int t = a0; t < A; t++) {
        double dot = 0.0;
        size_t kr = (size_t)kv_row(J, i, j, t);
        for (int x = 0; x < d; x++)
            dot += elem(J->q, qoff + x, J->q_dtype) * (ks * elem(J->k, kr + x, J->dtype));
        s[t] = J->scale * dot;
    }
    /* alpha_t = softmax_t(score); subtracting the max leaves it unchanged */
    double m = -INFINITY;
    for (int t = a0; t < A; t++)
        if (s[t] > m) m = s[t];
    double Z = 0.0;
    for (int t = a0; t < A; t++) {
        s[t] = exp(s[t] - m);
        Z += s[t];
    }
    for (int t = a0; t < A; t++) s[t] /= Z;
    /* O_i = sum_t alpha_t V_j,t */
    for (int x = 0; x < d; x++) {
        double acc = 0.0;
        for (int t = a0; t < A; t++)
            acc += s[t] * (vs * elem(J->v, (size_t)kv_row(J, i, j, t) + x, J->dtype));
        o[x] = acc;
    }
    if (J->alpha) {
        double *a = J->alpha + (size_t)row * S;
        for (int t = 0; t < S; t++) a[t] = (t >= a0 && t < A) ? s[t] : 0.0;
    }
    free(s);
}

static void *decode_worker(void *arg) {
    decode_job *J = (decode_job *)arg;
    for (int r = J->row_begin; r < J->row_end; r++) decode_row(J, r);
    return NULL;
}

/* Run the rows of a job template over nthreads POSIX threads. */
static int run_decode(const decode_job *tmpl, int nthreads) {
    int rows = tmpl->b * tmpl->T * tmpl->h;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > rows) nthreads = rows;
    decode_job *jobs = (decode_job *)calloc((size_t)nthreads, sizeof(decode_job));
    pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    for (int w = 0; w < nthreads; w++) {
        jobs[w] = *tmpl;
        jobs[w].row_begin = (int)((long)rows * w / nthreads);
        jobs[w].row_end = (int)((long)rows * (w + 1) / nthreads);
        jobs[w].flags = 0;
    }
    for (int w = 1; w < nthreads; w++)
        pthread_create(&tid[w], NULL, decode_worker, &jobs[w]);
    decode_worker(&jobs[0]);
    int rc = ORACLE_OK;
    for (int w = 0; w < nthreads; w++) {
        if (w) pthread_join(tid[w], NULL);
        rc |= jobs[w].flags;
    }
    free(jobs);
    free(tid);
    return rc;
}

int oracle_decode_attn_multi(const void *q, const void *k, const void *v,
                             const int32_t *seq_lens, int b, int T, int h, int g,
                             int S, int d, int dtype, float scale, double *out,
                             double *alpha, int nthreads) {
    if (b < 1 || T < 1 || h < 1 || g < 1 || S < 1 || d < 1 || h % g != 0)
        return ORACLE_BAD_SHAPE;
    decode_job J = {q, k, v, seq_lens, b, T, h, g, S, d, dtype, (double)scale,
                    out, alpha, 0, 0, 0, NULL, 0, 0, 0, dtype, NULL, NULL, 0};
    return run_decode(&J, nthreads);
}

int oracle_decode_attn(const void *q, const void *k, const void *v,
                       const int32_t *seq_lens, int b, int h, int g, int S,
                       int d, int dtype, float scale, double *out,
                       double *alpha, int nthreads) {
    return oracle_decode_attn_multi(q, k, v, seq_lens, b, 1, h, g, S, d, dtype,
                                    scale, out, alpha, nthreads);
}

int oracle_decode_attn_paged_multi(const void *q, const void *k_pages,
                                   const void *v_pages, const int32_t *block_table,
                                   const int32_t *seq_lens, int b, int T, int h,
                                   int g, int page_size, int max_pages,
                                   int num_pages, int d, int dtype, float scale,
                                   double *out, int nthreads) {
    if (b < 1 || T < 1 || h < 1 || g < 1 || d < 1 || h % g != 0 || page_size < 1 ||
        max_pages < 1 || num_pages < 1)
        return ORACLE_BAD_SHAPE;
    decode_job J = {q, k_pages, v_pages, seq_lens, b, T, h, g, page_size * max_pages,
                    d, dtype, (double)scale, out, NULL, 0, 0, 0, block_table,
                    page_size, max_pages, num_pages, dtype, NULL, NULL, 0};
    return run_decode(&J, nthreads);
}

int oracle_decode_attn_paged(const void *q, const void *k_pages,
                             const void *v_pages, const int32_t *block_table,
                             const int32_t *seq_lens, int b, int h, int g,
                             int page_size, int max_pages, int num_pages, int d,
                             int dtype, float scale, double *out, int nthreads) {
    return oracle_decode_attn_paged_multi(q, k_pages, v_pages, block_table, seq_lens,
                                          b, 1, h, g, page_size, max_pages,
                                          num_pages, d, dtype, scale, out, nthreads);
}

int oracle_append_kv_paged_multi(void *k_pages, void *v_pages, const void *k_new,
                                 const void *v_new, const int32_t *block_table,
                                 const int32_t *seq_lens, int b, int T, int g,
                                 int page_size, int max_pages, int num_pages, int d,
                                 int dtype) {
    if (b < 1 || T < 1 || g < 1 || d < 1 || page_size < 1 || max_pages < 1 ||
        num_pages < 1)
        return ORACLE_BAD_SHAPE;
    int rc = ORACLE_OK;
    size_t row = (size_t)d * elem_bytes(dtype);
    for (int i = 0; i < b; i++) {
        int L = seq_lens[i];
        if (L < T || L > page_size * max_pages) {
            rc |= ORACLE_BAD_LEN;
            continue;
        }
        for (int tau = 0; tau < T; tau++) {
            int t = L - T + tau; /* position of token tau */
            int page = block_table[(size_t)i * max_pages + t / page_size];
            if (page < 0 || page >= num_pages) {
                rc |= ORACLE_BAD_PAGE;
                continue;
            }
            for (int j = 0; j < g; j++) {
                size_t dst = (((size_t)page * g + j) * page_size + (size_t)(t % page_size)) * row;
                size_t src = (((size_t)i * T + tau) * g + j) * row;
                memcpy((char *)k_pages + dst, (const char *)k_new + src, row);
                memcpy((char *)v_pages + dst, (const char *)v_new + src, row);
            }
        }
    }
    return rc;
}

int oracle_append_kv_paged(void *k_pages, void *v_pages, const void *k_new,
                           const void *v_new, const int32_t *block_table,
                           const int32_t *seq_lens, int b, int g, int page_size,
                           int max_pages, int num_pages, int d, int dtype) {
    return oracle_append_kv_paged_multi(k_pages, v_pages, k_new, v_new, block_table,
                                        seq_lens, b, 1, g, page_size, max_pages,
                                        num_pages, d, dtype);
}

/* ---- textbook MHA, one K/V per query head ----------------------------- */

void oracle_mha_per_head(const double *q, const double *K, const double *V,
                         int h, int L, int d, double scale, double *out) {
    double *logits = (double *)malloc(sizeof(double) * (size_t)L);
    for (int hd = 0; hd < h; hd++) {
        const double *qh = q + (size_t)hd * d;
        const double *Kh = K + (size_t)hd * L * d;
        const double *Vh = V + (size_t)hd * L * d;
        double mx = -INFINITY;
        for (int t = 0; t < L; t++) {
            double acc = 0.0;
            for (int x = 0; x < d; x++) acc += qh[x] * Kh[(size_t)t * d + x];
            logits[t] = acc * scale;
            mx = fmax(mx, logits[t]);
        }
        double den = 0.0;
        for (int t = 0; t < L; t++) den += exp(logits[t] - mx);
        for (int x = 0; x < d; x++) {
            double num = 0.0;
            for (int t = 0; t < L; t++)
                num += exp(logits[t] - mx) * Vh[(size_t)t * d + x];
            out[(size_t)hd * d + x] = num / den;
        }
    }
    free(logits);
}

/* ---- shards and their log-sum-exp combination ------------------------ */

void oracle_partial(const double *q, const double *K, const double *V, int d,
                    double scale, int t0, int t1, double *m, double *l,
                    double *o) {
    for (int x = 0; x < d; x++) o[x] = 0.0;
    if (t1 <= t0) {
        *m = -INFINITY;
        *l = 0.0;
        return;
    }
    double mx = -INFINITY;
    for (int t = t0; t < t1; t++) {
        double s = 0.0;
        for (int x = 0; x < d; x++) s += q[x] * K[(size_t)t * d + x];
        mx = fmax(mx, s * scale);
    }
    double sum = 0.0;
    for (int t = t0; t < t1; t++) {
        double s = 0.0;
        for (int x = 0; x < d; x++) s += q[x] * K[(size_t)t * d + x];
        double w = exp(s * scale - mx);
        sum += w;
        for (int x = 0; x < d; x++) o[x] += w * V[(size_t)t * d + x];
    }
    *m = mx;
    *l = sum;
}

void oracle_lse_combine(int n, const double *m, const double *l,
                        const double *o, int d, double *out) {
    double M = -INFINITY;
    for (int s = 0; s < n; s++)
        if (l[s] > 0.0 && m[s] > M) M = m[s];
    double den = 0.0;
    for (int x = 0; x < d; x++) out[x] = 0.0;
    for (int s = 0; s < n; s++) {
        if (!(l[s] > 0.0)) continue;
        double w = exp(m[s] - M);
        den += w * l[s];
        for (int x = 0; x < d; x++) out[x] += w * o[(size_t)s * d + x];
    }
    for (int x = 0; x < d; x++) out[x] /= den;
}

uint64_t oracle_kv_bytes(int layers, int g, int64_t S, int d, int dtype_bytes) {
    return 2ull * (uint64_t)layers * (uint64_t)g * (uint64_t)S * (uint64_t)d *
           (uint64_t)dtype_bytes;
}

/* ---- fp8 e4m3 cache with per-K/V-head scales ------------------------------ */

int oracle_decode_attn_fp8(const void *q, int q_dtype, const uint8_t *k,
                           const uint8_t *v, const float *k_scale,
                           const float *v_scale, const int32_t *seq_lens, int b,
                           int T, int h, int g, int S, int d, float scale,
                           double *out, int nthreads) {
    if (b < 1 || T < 1 || h < 1 || g < 1 || S < 1 || d < 1 || h % g != 0)
        return ORACLE_BAD_SHAPE;
    decode_job J = {q, k, v, seq_lens, b, T, h, g, S, d, ORACLE_FP8_E4M3, (double)scale,
                    out, NULL, 0, 0, 0, NULL, 0, 0, 0, q_dtype, k_scale, v_scale, 0};
    return run_decode(&J, nthreads);
}

int oracle_decode_attn_paged_fp8(const void *q, int q_dtype, const uint8_t *k_pages,
                                 const uint8_t *v_pages, const float *k_scale,
                                 const float *v_scale, const int32_t *block_table,
                                 const int32_t *seq_lens, int b, int T, int h, int g,
                                 int page_size, int max_pages, int num_pages, int d,
                                 float scale, double *out, int nthreads) {
    if (b < 1 || T < 1 || h < 1 || g < 1 || d < 1 || h % g != 0 || page_size < 1 ||
        max_pages < 1 || num_pages < 1)
        return ORACLE_BAD_SHAPE;
    decode_job J = {q, k_pages, v_pages, seq_lens, b, T, h, g, page_size * max_pages, d,
                    ORACLE_FP8_E4M3, (double)scale, out, NULL, 0, 0, 0, block_table,
                    page_size, max_pages, num_pages, q_dtype, k_scale, v_scale, 0};
    return run_decode(&J, nthreads);
}

/* Code (of type `code`: fp8 e4m3 or int8) of one new element: its fp32
 * value divided by the head's scale (one correctly rounded fp32 division),
 * then encoded. */
static uint8_t quantise(const void *src, size_t idx, int dtype, float scale, int code) {
    float x = (float)elem(src, idx, dtype); /* exact: the source is f32 or bf16 */
    float y = x / scale;
    if (code == ORACLE_INT8) return (uint8_t)oracle_int8_encode(y);
    return oracle_fp8_e4m3_encode(y);
}

static int append_codes(uint8_t *k_cache, uint8_t *v_cache, const void *k_new,
                        const void *v_new, int new_dtype, const float *k_scale,
                        const float *v_scale, const int32_t *seq_lens, int b, int T, int g,
                        int S, int d, int code) {
    if (b < 1 || T < 1 || g < 1 || S < 1 || d < 1) return ORACLE_BAD_SHAPE;
    int rc = ORACLE_OK;
    for (int i = 0; i < b; i++) {
        int L = seq_lens[i];
        if (L < T || L > S) {
            rc |= ORACLE_BAD_LEN;
            continue;
        }
        for (int tau = 0; tau < T; tau++)
            for (int j = 0; j < g; j++) {
                size_t dst = (((size_t)i * g + j) * S + (size_t)(L - T + tau)) * d;
                size_t src = (((size_t)i * T + tau) * g + j) * d;
                for (int x = 0; x < d; x++) {
                    k_cache[dst + x] = quantise(k_new, src + x, new_dtype, k_scale[j], code);
                    v_cache[dst + x] = quantise(v_new, src + x, new_dtype, v_scale[j], code);
                }
            }
    }
    return rc;
}

static int append_codes_paged(uint8_t *k_pages, uint8_t *v_pages, const void *k_new,
                              const void *v_new, int new_dtype, const float *k_scale,
                              const float *v_scale, const int32_t *block_table,
                              const int32_t *seq_lens, int b, int T, int g, int page_size,
                              int max_pages, int num_pages, int d, int code) {
    if (b < 1 || T < 1 || g < 1 || d < 1 || page_size < 1 || max_pages < 1 || num_pages < 1)
        return ORACLE_BAD_SHAPE;
    int rc = ORACLE_OK;
    for (int i = 0; i < b; i++) {
        int L = seq_lens[i];
        if (L < T || L > page_size * max_pages) {
            rc |= ORACLE_BAD_LEN;
            continue;
        }
        for (int tau = 0; tau < T; tau++) {
            int t = L - T + tau;
            int page = block_table[(size_t)i * max_pages + t / page_size];
            if (page < 0 || page >= num_pages) {
                rc |= ORACLE_BAD_PAGE;
                continue;
            }
            for (int j = 0; j < g; j++) {
                size_t dst = (((size_t)page * g + j) * page_size + (size_t)(t % page_size)) * d;
                size_t src = (((size_t)i * T + tau) * g + j) * d;
                for (int x = 0; x < d; x++) {
                    k_pages[dst + x] = quantise(k_new, src + x, new_dtype, k_scale[j], code);
                    v_pages[dst + x] = quantise(v_new, src + x, new_dtype, v_scale[j], code);
                }
            }
        }
    }
    return rc;
}

int oracle_append_kv_fp8(uint8_t *k_cache, uint8_t *v_cache, const void *k_new,
                         const void *v_new, int new_dtype, const float *k_scale,
                         const float *v_scale, const int32_t *seq_lens, int b, int T,
                         int g, int S, int d) {
    return append_codes(k_cache, v_cache, k_new, v_new, new_dtype, k_scale, v_scale, seq_lens,
                        b, T, g, S, d, ORACLE_FP8_E4M3);
}

int oracle_append_kv_paged_fp8(uint8_t *k_pages, uint8_t *v_pages, const void *k_new,
                               const void *v_new, int new_dtype, const float *k_scale,
                               const float *v_scale, const int32_t *block_table,
                               const int32_t *seq_lens, int b, int T, int g, int page_size,
                               int max_pages, int num_pages, int d) {
    return append_codes_paged(k_pages, v_pages, k_new, v_new, new_dtype, k_scale, v_scale,
                              block_table, seq_lens, b, T, g, page_size, max_pages, num_pages, d,
                              ORACLE_FP8_E4M3);
}

int oracle_append_kv_int8(int8_t *k_cache, int8_t *v_cache, const void *k_new,
                          const void *v_new, int new_dtype, const float *k_scale,
                          const float *v_scale, const int32_t *seq_lens, int b, int T,
                          int g, int S, int d) {
    return append_codes((uint8_t *)k_cache, (uint8_t *)v_cache, k_new, v_new, new_dtype,
                        k_scale, v_scale, seq_lens, b, T, g, S, d, ORACLE_INT8);
}

int oracle_append_kv_paged_int8(int8_t *k_pages, int8_t *v_pages, const void *k_new,
                                const void *v_new, int new_dtype, const float *k_scale,
                                const float *v_scale, const int32_t *block_table,
                                const int32_t *seq_lens, int b, int T, int g, int page_size,
                                int max_pages, int num_pages, int d) {
    return append_codes_paged((uint8_t *)k_pages, (uint8_t *)v_pages, k_new, v_new, new_dtype,
                              k_scale, v_scale, block_table, seq_lens, b, T, g, page_size,
                              max_pages, num_pages, d, ORACLE_INT8);
}

/* ---- every option at once: layout, cache element type, tokens, window ---- */

int oracle_decode_attn_ex(const void *q, int q_dtype, const void *k, const void *v,
                          int kv_dtype, const float *k_scale, const float *v_scale,
                          const int32_t *block_table, int page_size, int max_pages,
                          int num_pages, const int32_t *seq_lens, int b, int T, int h, int g,
                          int S, int d, int window, float scale, double *out, int nthreads) {
    if (b < 1 || T < 1 || h < 1 || g < 1 || d < 1 || h % g != 0 || window < 0)
        return ORACLE_BAD_SHAPE;
    if (block_table) {
        if (page_size < 1 || max_pages < 1 || num_pages < 1) return ORACLE_BAD_SHAPE;
        S = page_size * max_pages;
    } else if (S < 1) {
        return ORACLE_BAD_SHAPE;
    }
    decode_job J = {q, k, v, seq_lens, b, T, h, g, S, d, kv_dtype, (double)scale, out, NULL,
                    0, 0, 0, block_table, page_size, max_pages, num_pages, q_dtype,
                    k_scale, v_scale, window};
    return run_decode(&J, nthreads);
}

/* ---- rotary position embedding (RoPE) -------------------------------------- */

/* cos_sin[p][i] = (cos(p * th_i), sin(p * th_i)) rounded to fp32, th_i =
 * base^(-2i/d), i < d/2: the rotation angles of position p (computed in
 * double). */
void oracle_rope_table(double base, int n_pos, int d, float *cos_sin) {
    for (int p = 0; p < n_pos; p++)
        for (int i = 0; i < d / 2; i++) {
            double th = pow(base, -2.0 * i / d);
            cos_sin[((size_t)p * (d / 2) + i) * 2 + 0] = (float)cos(p * th);
            cos_sin[((size_t)p * (d / 2) + i) * 2 + 1] = (float)sin(p * th);
        }
}

/* Nearest bf16 of a float (ties to even; NaN kept). */
static uint16_t bf16_round(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

/* Rotate one bf16 row of d elements at position pos: element i and element
 * i + d/2 form a pair (the halves convention), turned by the angle of pair
 * i: a' = a c - b s, b' = b c + a s, each product and the sum rounded to fp32
 * in that order (no fused multiply-add), the results rounded to bf16. */
static void rope_row(uint16_t *row, int pos, const float *cos_sin, int d) {
    int hd = d / 2;
    for (int i = 0; i < hd; i++) {
        float a = (float)elem(row, (size_t)i, ORACLE_BF16);
        float b = (float)elem(row, (size_t)(i + hd), ORACLE_BF16);
        float c = cos_sin[((size_t)pos * hd + i) * 2 + 0];
        float s = cos_sin[((size_t)pos * hd + i) * 2 + 1];
        float ac = a * c, bs = b * s, bc = b * c, as = a * s;
        float ra = ac - bs, rb = bc + as;
        row[i] = bf16_round(ra);
        row[i + hd] = bf16_round(rb);
    }
}

/* In place: rows x [n][d] (bf16 bits) rotated at positions pos[n]. */
void oracle_rope_rows(uint16_t *x, const int32_t *pos, const float *cos_sin, int n, int d) {
    for (int r = 0; r < n; r++) rope_row(x + (size_t)r * d, pos[r], cos_sin, d);
}

/* q [b][T][h][d] (bf16) rotated in place: token tau of sequence i at
 * position L_i - T + tau. Sequences with a bad length are left alone. */
int oracle_rope_q(uint16_t *q, const float *cos_sin, const int32_t *seq_lens, int b, int T,
                  int h, int d) {
    int rc = ORACLE_OK;
    for (int i = 0; i < b; i++) {
        int L = seq_lens[i];
        if (L < T) {
            rc |= ORACLE_BAD_LEN;
            continue;
        }
        for (int tau = 0; tau < T; tau++)
            for (int hq = 0; hq < h; hq++)
                rope_row(q + (((size_t)i * T + tau) * h + hq) * d, L - T + tau, cos_sin, d);
    }
    return rc;
}

/* Append with RoPE on K ([GQA notes] §十 item 6: the rotation is applied
 * per head, to each K/V head's key as to each query head's query): token
 * tau's key row, rotated at its position L - T + tau, and its value row, as
 * is, go to that position (bf16 cache [b][g][S][d]; k_new, v_new
 * [b][T][g][d]). */
int oracle_append_kv_rope(uint16_t *k_cache, uint16_t *v_cache, const uint16_t *k_new,
                          const uint16_t *v_new, const float *cos_sin,
                          const int32_t *seq_lens, int b, int T, int g, int S, int d) {
    int rc = oracle_append_kv_multi(k_cache, v_cache, k_new, v_new, seq_lens, b, T, g, S, d,
                                    ORACLE_BF16);
    if (rc == ORACLE_BAD_SHAPE) return rc;
    for (int i = 0; i < b; i++) {
        int L = seq_lens[i];
        if (L < T || L > S) continue;
        for (int tau = 0; tau < T; tau++)
            for (int j = 0; j < g; j++)
                rope_row(k_cache + (((size_t)i * g + j) * S + (size_t)(L - T + tau)) * d,
                         L - T + tau, cos_sin, d);
    }
    return rc;
}

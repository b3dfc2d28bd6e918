/*
 * Plain CPU oracle for decode attention over a shared-head KV cache.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link,
 * load or call this code: only the tests, the smoke check and the bench's
 * CPU-baseline leg use it. It shares no header, table or helper with the HIP
 * library, and it is written for obviousness, not speed: double precision,
 * plain loops, no blocking, fusion or reordering beyond what the definitions
 * state.
 *
 * Sources (web pages, cited by title and section):
 *  [GQA notes]  ybb.press, "分组查询注意力（GQA）与多查询注意力（MQA）深度实战"
 *               §一 (KV bytes), §四 (GQA grouping), §五 (math form), §七 (h/g),
 *               §八 (reference implementation: cache write, repeat_interleave).
 *  [MQA blog]   nanhubrain.csdn.net MQA article, §2.2 (concat of the new K/V on
 *               the sequence axis), §3.3 (paged cache, 16 tokens per page).
 *  [MQA concept] compassingai.com "多查詢注意力", 技術原理 / "KV Cache 結構與
 *               視訊記憶體佔用對比" (per-layer byte counts).
 *
 * Element types: ORACLE_F32 is IEEE binary32; ORACLE_BF16 is bfloat16, i.e.
 * the upper 16 bits of a binary32 (decoded exactly by a 16-bit shift).
 *
 * Layouts (row-major, last index fastest):
 *   q        [b][h][d]        ([b][T][h][d] for T query tokens per sequence)
 *   k, v     [b][g][S][d]     (S = capacity; rows >= seq_lens[i] are unused)
 *   k/v_new  [b][g][d]        ([b][T][g][d])
 *   out      [b][h][d]        (double; [b][T][h][d])
 *   alpha    [b][h][S]        (double, optional attention weights; [b][T][h][S])
 */
#ifndef ORACLE_DECODE_ATTN_H
#define ORACLE_DECODE_ATTN_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_FP8_E4M3 = 2, ORACLE_INT8 = 3 };

/* Return bits. ORACLE_BAD_LEN: some seq_lens[i] outside [1, S] ([T, S] with T
 * query tokens); those rows
 * are left alone by append and set to NaN by decode. ORACLE_BAD_SHAPE: h not a
 * multiple of g, or a size < 1; nothing is written. */
enum { ORACLE_OK = 0, ORACLE_BAD_LEN = 1, ORACLE_BAD_SHAPE = 2, ORACLE_BAD_PAGE = 4 };

/* Cache append: row seq_lens[i]-1 of every K/V head j of sequence i receives
 * k_new[i][j][:] / v_new[i][j][:], byte for byte. [MQA blog] §2.2;
 * [GQA notes] §八 (cache_k[:, start:start+T] = k). */
int oracle_append_kv(void *k_cache, void *v_cache, const void *k_new,
                     const void *v_new, const int32_t *seq_lens, int b, int g,
                     int S, int d, int dtype);

/* Decode attention, the plain definition ([GQA notes] §四, §五):
 *   j = hq / (h/g);  score_t = scale * q[i,hq,:].k[i,j,t,:]   for t < L_i
 *   alpha_t = softmax_t(score);  out[i,hq,:] = sum_t alpha_t v[i,j,t,:]
 * nthreads >= 1 splits the (i, hq) rows across POSIX threads; each row is
 * computed by the same loop either way. */
int oracle_decode_attn(const void *q, const void *k, const void *v,
                       const int32_t *seq_lens, int b, int h, int g, int S,
                       int d, int dtype, float scale, double *out,
                       double *alpha, int nthreads);

/* Paged cache ([MQA blog] §3.3: the cache cut into fixed-size pages, 16
 * tokens by default; [GQA notes] §十 item 12: ragged batches managed with
 * pages): K/V live in pages k_pages, v_pages [num_pages][g][page_size][d];
 * position t of sequence i is row t % page_size of page
 * block_table[i][t / page_size] (block_table [b][max_pages], int32).
 * Decode is the plain definition above over the positions t < L_i looked up
 * this way; a row that reads a page id outside [0, num_pages) is NaN and
 * ORACLE_BAD_PAGE is returned. Append writes row (L_i-1) % page_size of page
 * block_table[i][(L_i-1) / page_size]. Capacity is page_size * max_pages. */
int oracle_decode_attn_paged(const void *q, const void *k_pages,
                             const void *v_pages, const int32_t *block_table,
                             const int32_t *seq_lens, int b, int h, int g,
                             int page_size, int max_pages, int num_pages, int d,
                             int dtype, float scale, double *out, int nthreads);
int oracle_append_kv_paged(void *k_pages, void *v_pages, const void *k_new,
                           const void *v_new, const int32_t *block_table,
                           const int32_t *seq_lens, int b, int g, int page_size,
                           int max_pages, int num_pages, int d, int dtype);

/* T query tokens per sequence (a draft of several tokens verified at once,
 * or a chunk of a prompt): the step's tokens are positions L_i-T .. L_i-1
 * (seq_lens counts them), token tau attends positions t <= L_i-T+tau only,
 * since the causal mask is applied per query position whether K/V are shared
 * or not ([GQA notes] §十 item 10; the §八 reference code writes T rows at
 * once). Rows of q and out are (i*T + tau)*h + hq. seq_lens[i] < T is a bad
 * length. Append writes token tau of k_new/v_new [b][T][g][d] to position
 * L_i-T+tau. T = 1 is the functions above, which call these. */
int oracle_append_kv_multi(void *k_cache, void *v_cache, const void *k_new,
                           const void *v_new, const int32_t *seq_lens, int b,
                           int T, int g, int S, int d, int dtype);
int oracle_decode_attn_multi(const void *q, const void *k, const void *v,
                             const int32_t *seq_lens, int b, int T, int h, int g,
                             int S, int d, int dtype, float scale, double *out,
                             double *alpha, int nthreads);
int oracle_decode_attn_paged_multi(const void *q, const void *k_pages,
                                   const void *v_pages, const int32_t *block_table,
                                   const int32_t *seq_lens, int b, int T, int h,
                                   int g, int page_size, int max_pages,
                                   int num_pages, int d, int dtype, float scale,
                                   double *out, int nthreads);
int oracle_append_kv_paged_multi(void *k_pages, void *v_pages, const void *k_new,
                                 const void *v_new, const int32_t *block_table,
                                 const int32_t *seq_lens, int b, int T, int g,
                                 int page_size, int max_pages, int num_pages, int d,
                                 int dtype);

/* Low-precision cache ([GQA notes] §十 item 7: a quantised KV cache stacks
 * with grouping but must be validated on its own): K and V held as fp8 e4m3
 * codes (OCP E4M3FN: bias 7, 3 mantissa bits, no infinity, largest finite
 * 448), one scale per K/V head for K and one for V (k_scale, v_scale [g],
 * fp32); a cache value is code * scale[j]. Decode is the plain definition
 * (the T-token form above, q of q_dtype [b][T][h][d]) over those values.
 * Append: each new element x (k_new, v_new [b][T][g][d] of new_dtype) is
 * stored as encode(x / scale[j]), the division one correctly rounded fp32
 * operation and the encoding round-to-nearest-even with saturation at
 * +-448 (a finite value never becomes NaN). */
double oracle_fp8_e4m3_decode(uint8_t code);
uint8_t oracle_fp8_e4m3_encode(float x);
int oracle_decode_attn_fp8(const void *q, int q_dtype, const uint8_t *k,
                           const uint8_t *v, const float *k_scale,
                           const float *v_scale, const int32_t *seq_lens, int b,
                           int T, int h, int g, int S, int d, float scale,
                           double *out, int nthreads);
int oracle_decode_attn_paged_fp8(const void *q, int q_dtype, const uint8_t *k_pages,
                                 const uint8_t *v_pages, const float *k_scale,
                                 const float *v_scale, const int32_t *block_table,
                                 const int32_t *seq_lens, int b, int T, int h, int g,
                                 int page_size, int max_pages, int num_pages, int d,
                                 float scale, double *out, int nthreads);
int oracle_append_kv_fp8(uint8_t *k_cache, uint8_t *v_cache, const void *k_new,
                         const void *v_new, int new_dtype, const float *k_scale,
                         const float *v_scale, const int32_t *seq_lens, int b, int T,
                         int g, int S, int d);
int oracle_append_kv_paged_fp8(uint8_t *k_pages, uint8_t *v_pages, const void *k_new,
                               const void *v_new, int new_dtype, const float *k_scale,
                               const float *v_scale, const int32_t *block_table,
                               const int32_t *seq_lens, int b, int T, int g, int page_size,
                               int max_pages, int num_pages, int d);

/* int8 cache (the other low-precision format the pages name: [MQA concept]'s
 * risk list and [MQA blog] §4.3 problem 3 speak of INT8/INT4 K/V). Codes are
 * two's-complement int8 with the same per-K/V-head scales as the fp8 cache
 * (value = code * scale[j]); decode is the plain definition over those
 * values (oracle_decode_attn_ex with kv_dtype ORACLE_INT8). Append stores
 * encode(x / scale[j]): one correctly rounded fp32 division, then the
 * nearest integer, ties to even, saturated at +-127 (never -128: the codes
 * are symmetric about 0); NaN becomes 0. */
double oracle_int8_decode(int8_t code);
int8_t oracle_int8_encode(float x);
int oracle_append_kv_int8(int8_t *k_cache, int8_t *v_cache, const void *k_new,
                          const void *v_new, int new_dtype, const float *k_scale,
                          const float *v_scale, const int32_t *seq_lens, int b, int T,
                          int g, int S, int d);
int oracle_append_kv_paged_int8(int8_t *k_pages, int8_t *v_pages, const void *k_new,
                                const void *v_new, int new_dtype, const float *k_scale,
                                const float *v_scale, const int32_t *block_table,
                                const int32_t *seq_lens, int b, int T, int g, int page_size,
                                int max_pages, int num_pages, int d);

/* Every option of the decode at once: q (q_dtype) [b][T][h][d]; K/V
 * contiguous [b][g][S][d] (block_table NULL) or pages [num_pages][g][P][d]
 * through block_table [b][max_pages] (S is then P * max_pages); kv_dtype
 * f32, bf16, fp8 e4m3 or int8 (codes with k_scale, v_scale [g]; NULL
 * otherwise); a
 * sliding window: window > 0 keeps, for a query at position p, only the
 * positions t in (p - window, p] (the window start replaces 0: [MQA
 * concept] 玩家對比 lists GQA with a sliding window); 0 keeps all t <= p. */
int oracle_decode_attn_ex(const void *q, int q_dtype, const void *k, const void *v,
                          int kv_dtype, const float *k_scale, const float *v_scale,
                          const int32_t *block_table, int page_size, int max_pages,
                          int num_pages, const int32_t *seq_lens, int b, int T, int h, int g,
                          int S, int d, int window, float scale, double *out, int nthreads);

/* Rotary position embedding on bf16 rows ([GQA notes] §十 item 6: position
 * information is applied per head, to queries and to each K/V head's keys
 * alike; the pages give no formula, so the common rotary form): pairs
 * (x_i, x_{i+d/2}), i < d/2, are turned by the angle p * base^(-2i/d) of
 * position p. oracle_rope_table writes cos_sin [n_pos][d/2][2] fp32 (cos,
 * sin) from the angles in double. The rotation of a pair is a' = a c - b s,
 * b' = b c + a s in fp32 (each product rounded, then the sum, no fused
 * multiply-add), rounded to bf16 (nearest, ties to even). */
void oracle_rope_table(double base, int n_pos, int d, float *cos_sin);
void oracle_rope_rows(uint16_t *x, const int32_t *pos, const float *cos_sin, int n, int d);
int oracle_rope_q(uint16_t *q, const float *cos_sin, const int32_t *seq_lens, int b, int T,
                  int h, int d);
int oracle_append_kv_rope(uint16_t *k_cache, uint16_t *v_cache, const uint16_t *k_new,
                          const uint16_t *v_new, const float *cos_sin,
                          const int32_t *seq_lens, int b, int T, int g, int S, int d);

/* Textbook multi-head attention for one sequence, one K/V head per query
 * head (no sharing): q [h][d], K and V [h][L][d], all double.
 * [GQA notes] §二: O_i = softmax(Q_i K_i^T / sqrt(d_h)) V_i. */
void oracle_mha_per_head(const double *q, const double *K, const double *V,
                         int h, int L, int d, double scale, double *out);

/* One shard [t0, t1) of one query row: m = max score, l = sum exp(s - m),
 * o[:] = sum exp(s - m) v[t,:] (unnormalised). q [d], K and V [L][d] double. */
void oracle_partial(const double *q, const double *K, const double *V, int d,
                    double scale, int t0, int t1, double *m, double *l,
                    double *o);

/* Log-sum-exp combine of n shards (m[s], l[s], o[s][d]) into out[d]:
 * M = max m_s, out = sum_s e^(m_s-M) o_s / sum_s e^(m_s-M) l_s.
 * Shards with l == 0 (empty) are skipped. */
void oracle_lse_combine(int n, const double *m, const double *l,
                        const double *o, int d, double *out);

/* KV-cache bytes, [GQA notes] §一 and §七: 2 * layers * g * S * d * bytes. */
uint64_t oracle_kv_bytes(int layers, int g, int64_t S, int d, int dtype_bytes);

#ifdef __cplusplus
}
#endif
#endif

/*
 * mqa_decode.h - C ABI of the MI355X (gfx950) decode-attention library
 * libmqa_decode.so: one autoregressive decode step over a KV cache in which
 * h query heads share g K/V heads (g = 1: multi-query, 1 < g < h: grouped-
 * query, g = h: multi-head attention).
 *
 * Sources, cited by page title and section:
 *  [GQA notes]   ybb.press, "分组查询注意力（GQA）与多查询注意力（MQA）深度实战":
 *                §一 and §七 (KV-cache bytes and the h/g ratio), §四 (g groups,
 *                g divides h), §五 (head-to-group map j = i // (h/g), score,
 *                softmax, weighted sum), §八 (preallocated cache of capacity
 *                max_seq written at the current position), §十 (pitfalls:
 *                divisibility, ragged batches).
 *  [MQA blog]    nanhubrain.csdn.net MQA article: §2.2 (the new K/V is
 *                concatenated onto the cache along the sequence axis), §4.3
 *                (capacity overflow must not truncate silently).
 *  [MQA concept] compassingai.com "多查詢注意力", 技術原理 (per-layer bytes).
 *
 * Conventions shared by every entry point
 *  - Tensors are contiguous, row-major, last index fastest, in device memory
 *    owned by the caller. The library allocates nothing and never
 *    synchronises: work is enqueued on `stream` (a hipStream_t; NULL is the
 *    default stream) and completes in stream order. Its only global state is
 *    mqa_decode_attn_noalloc's scratch array and that array's address per
 *    device (see there); every other call keeps none.
 *  - Element type `dt` applies to q, k_cache, v_cache, k_new and v_new.
 *    MQA_BF16 is bfloat16 (upper 16 bits of a binary32). Outputs are fp32.
 *  - d (head dimension) is 64 or 128. Every tensor pointer must be 16-byte
 *    aligned (the kernels use 128-bit loads).
 *  - seq_lens[b] (device, int32) holds, for each sequence, the number of
 *    positions attended INCLUDING the token appended this step; the append
 *    writes cache row seq_lens[i]-1.
 *  - Host-detectable argument errors return a status before anything is
 *    enqueued. A HIP launch failure returns MQA_ERR_HIP.
 *  - Device-detectable errors never truncate silently: a sequence whose
 *    seq_lens[i] is outside [1, S] is skipped by the append, gets NaN in every
 *    element of out[i,:,:] from the decode, and both OR MQA_DEVERR_SEQLEN into
 *    *err_flags when err_flags is non-NULL (a device int32 the caller clears).
 */
#ifndef MQA_DECODE_H
#define MQA_DECODE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MQA_OK = 0,
    MQA_ERR_NULL = 1,        /* a required pointer is NULL */
    MQA_ERR_SHAPE = 2,       /* a size < 1, h not a multiple of g, b > 65535,
                                g*h > 2^30, or one K/V head's S rows
                                (S*d*elem) >= 2 GiB */
    MQA_ERR_UNSUPPORTED = 3, /* d not 64/128, unknown dtype, bad split_chunk */
    MQA_ERR_ALIGN = 4,       /* a tensor pointer not 16-byte aligned */
    MQA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required */
    MQA_ERR_HIP = 6,         /* the HIP runtime reported a launch error */
    MQA_ERR_SCRATCH = 7,     /* mqa_decode_attn_noalloc: the call needs more
                                scratch than the library's array holds */
    /* (the two bounds below only pin each enum of this header to the range
     * of int, so that any int a caller passes is a value of the type: an
     * invalid one then gets the documented error status, where a value
     * outside an enum's range would be undefined behaviour in C++) */
    MQA_STATUS_INT_MIN_ = -2147483647 - 1,
    MQA_STATUS_INT_MAX_ = 2147483647
} mqa_status;

/* Element types. MQA_FP8_E4M3 and MQA_INT8 are cache types only
 * (mqa_decode_attn_ex, the _fp8 and _int8 calls); q and new rows are then
 * bf16. */
typedef enum {
    MQA_F32 = 0,
    MQA_BF16 = 1,
    MQA_FP8_E4M3 = 2,
    MQA_INT8 = 3,
    MQA_DTYPE_INT_MIN_ = -2147483647 - 1, /* range of int (see mqa_status) */
    MQA_DTYPE_INT_MAX_ = 2147483647
} mqa_dtype;

/* Which partition kernel computes the attention (see mqa_decode_attn_kernel). */
typedef enum {
    MQA_KERNEL_AUTO = 0, /* bf16: matrix cores; fp32: vector ALUs */
    MQA_KERNEL_VALU = 1, /* vector-ALU kernel (bf16 dot2 / fp32 FMA), any dtype */
    MQA_KERNEL_MFMA = 2, /* matrix-core kernel, bf16 only */
    /* matrix-core kernel, bf16 only, with results bitwise identical call
     * after call: on the balanced schedule each wave takes a fixed share of
     * its work-group's steps (dealt round robin in claim order) instead of
     * claiming them as it goes, and a segment's states are merged in wave
     * order; the fixed partitions already repeat bit for bit. Slower where
     * the waves' memory service is uneven. */
    MQA_KERNEL_MFMA_DETERMINISTIC = 3,
    MQA_KERNEL_INT_MIN_ = -2147483647 - 1, /* range of int (see mqa_status) */
    MQA_KERNEL_INT_MAX_ = 2147483647
} mqa_kernel;

/* Bits ORed into *err_flags by the kernels: some seq_lens[i] outside [1, S];
 * some position of a paged call on a page id outside [0, num_pages); some
 * position of a rotary call past the rows of its cos/sin table. */
#define MQA_DEVERR_SEQLEN 1
#define MQA_DEVERR_PAGE 2
#define MQA_DEVERR_ROPE 4
/* A wait between the waves of one work-group of the balanced schedule ran
 * past its bound (a failure of the claim protocol, which a CPU model of it in
 * the tests rules out): that work-group's rows are NaN, nothing hangs. */
#define MQA_DEVERR_STALL 8

/*
 * Append this step's K/V rows to the cache, bit-exactly.
 * [MQA blog] §2.2 (concat on the sequence axis); [GQA notes] §八 (cache
 * written at the current position of a preallocated max_seq buffer).
 *
 *   k_cache, v_cache : [b][g][S][d] of dt, updated in place
 *   k_new, v_new     : [b][g][d]    of dt
 *   seq_lens         : [b] int32 device, post-append lengths
 * For every i < b with 1 <= seq_lens[i] <= S and every j < g:
 *   k_cache[i][j][seq_lens[i]-1][:] = k_new[i][j][:]   (same for v)
 * No other byte of the caches is written.
 */
mqa_status mqa_append_kv(void *k_cache, void *v_cache, const void *k_new,
                         const void *v_new, const int32_t *seq_lens, int b,
                         int g, int S, int d, mqa_dtype dt, int32_t *err_flags,
                         hipStream_t stream);

/*
 * Bytes of device workspace mqa_decode_attn needs for these sizes and this
 * split_chunk (0 = automatic). Returns 0 if the arguments are invalid.
 */
size_t mqa_decode_workspace_bytes(int b, int h, int g, int S, int d,
                                  mqa_dtype dt, int split_chunk);

/*
 * The sequence-split length (positions per partition) mqa_decode_attn uses
 * for these sizes: split_chunk itself when non-zero, else the automatic
 * choice. Returns -1 if the arguments are invalid.
 */
int mqa_decode_resolve_chunk(int b, int h, int g, int S, int d, mqa_dtype dt,
                             int split_chunk);

/*
 * Decode attention for one step. [GQA notes] §四/§五: for query head hq of
 * sequence i, with G = h/g and j = hq / G,
 *   score_t = scale * q[i][hq][:] . k_cache[i][j][t][:],   0 <= t < seq_lens[i]
 *   out[i][hq][:] = sum_t softmax_t(score)_t * v_cache[i][j][t][:]
 * Cache rows t >= seq_lens[i] are never read into the result (they may hold
 * anything, NaN included).
 *
 *   q                : [b][h][d] of dt
 *   k_cache, v_cache : [b][g][S][d] of dt (read only)
 *   seq_lens         : [b] int32 device
 *   scale            : score scale, normally 1/sqrt(d)
 *   out              : [b][h][d] fp32, fully overwritten
 *   workspace        : >= mqa_decode_workspace_bytes(...) bytes of device
 *                      memory, 16-byte aligned, for partial results; its
 *                      contents on entry are ignored.
 *   split_chunk      : positions per partition, a multiple of 64, or 0 for
 *                      the automatic choice
 * The sequence is cut into partitions; each keeps a running max and sum
 * (online softmax) and a log-sum-exp merge combines them. With split_chunk
 * > 0 the partitions are split_chunk positions long; with 0 the library
 * chooses, and for bf16 batches of many (sequence, K/V head) pairs it splits
 * the total work evenly over the compute units whatever the lengths.
 * Concurrent calls must not share a workspace.
 */
mqa_status mqa_decode_attn(const void *q, const void *k_cache,
                           const void *v_cache, const int32_t *seq_lens, int b,
                           int h, int g, int S, int d, mqa_dtype dt,
                           float scale, float *out, void *workspace,
                           size_t workspace_bytes, int split_chunk,
                           int32_t *err_flags, hipStream_t stream);

/*
 * mqa_decode_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops and harnesses that forbid hipMalloc): the
 * same arguments, kernels and results without the workspace, whose partials
 * go to a scratch array of 64 MiB that the library holds on each GPU it runs
 * on until the process ends. The call allocates nothing and uses the current
 * device's array (`stream` must belong to the current device); the array's
 * address is looked up once per device, on the first call there (make that
 * first call outside graph capture). Calls that need more than 64 MiB of
 * workspace (mqa_decode_workspace_bytes) return MQA_ERR_SCRATCH before
 * anything is enqueued. Every call on a GPU shares that GPU's array, which
 * keeps the last call's contents (nothing in it needs to start at zero):
 * calls that overlap on one GPU (other streams, other host threads) race.
 */
mqa_status mqa_decode_attn_noalloc(const void *q, const void *k_cache,
                                   const void *v_cache, const int32_t *seq_lens,
                                   int b, int h, int g, int S, int d,
                                   mqa_dtype dt, float scale, float *out,
                                   int split_chunk, int32_t *err_flags,
                                   hipStream_t stream);

/*
 * mqa_decode_attn with an explicit choice of partition kernel; same arguments,
 * layouts, workspace and results (to floating-point rounding). MQA_KERNEL_MFMA
 * and MQA_KERNEL_MFMA_DETERMINISTIC with dt = MQA_F32 return
 * MQA_ERR_UNSUPPORTED. mqa_decode_attn is this call with MQA_KERNEL_AUTO,
 * whose balanced schedule lets waves claim steps as they go: which wave sums
 * which steps then varies with timing, and so do the last bits of the sums
 * (within the bound stated with the tests; the fixed partitions repeat bit
 * for bit).
 */
mqa_status mqa_decode_attn_kernel(const void *q, const void *k_cache,
                                  const void *v_cache, const int32_t *seq_lens,
                                  int b, int h, int g, int S, int d,
                                  mqa_dtype dt, float scale, float *out,
                                  void *workspace, size_t workspace_bytes,
                                  int split_chunk, int32_t *err_flags,
                                  mqa_kernel kernel, hipStream_t stream);

/* The schedule mqa_decode_attn_kernel runs for these arguments. */
typedef enum {
    MQA_SCHEDULE_VALU_PARTITIONS = 0, /* vector-ALU partition kernel + combine kernel */
    MQA_SCHEDULE_MFMA_PARTITIONS = 1, /* matrix-core partition kernel + combine kernel */
    MQA_SCHEDULE_MFMA_BALANCED = 2    /* matrix-core kernel with equal work per
                                         compute unit + a merge kernel for the
                                         units cut between work-groups */
} mqa_schedule;

/* Which schedule (above) a call with these arguments runs; -1 if the
 * arguments are invalid. Host only, enqueues nothing. */
int mqa_decode_schedule(int b, int h, int g, int S, int d, mqa_dtype dt,
                        int split_chunk, mqa_kernel kernel);

/*
 * Paged KV cache. [MQA blog] §3.3 (the cache cut into fixed-size pages, 16
 * tokens by default); [GQA notes] §十 item 12 (ragged batches managed with
 * pages rather than padding).
 *
 *   k_pages, v_pages : [num_pages][g][page_size][d] of dt
 *   block_table      : [b][max_pages] int32 device: the page ids of sequence
 *                      i in position order; position t of sequence i is row
 *                      t % page_size of page block_table[i][t / page_size].
 *                      Entries past the length are never read; pages may be
 *                      shared between sequences (a common prefix).
 * Capacity S = page_size * max_pages; seq_lens as above (post-append).
 * page_size is a positive multiple of 16. The decode is bf16 only
 * (MQA_F32 returns MQA_ERR_UNSUPPORTED) and runs the matrix-core kernels.
 * A position on a page id outside [0, num_pages) gives NaN rows for its
 * sequence's query heads of that K/V head (decode) or skips the row (append)
 * and ORs MQA_DEVERR_PAGE into *err_flags.
 */
mqa_status mqa_append_kv_paged(void *k_pages, void *v_pages, const void *k_new,
                               const void *v_new, const int32_t *block_table,
                               const int32_t *seq_lens, int b, int g,
                               int page_size, int max_pages, int num_pages,
                               int d, mqa_dtype dt, int32_t *err_flags,
                               hipStream_t stream);

/* Bytes of workspace mqa_decode_attn_paged needs (0: invalid arguments). */
size_t mqa_decode_paged_workspace_bytes(int b, int h, int g, int page_size,
                                        int max_pages, int d, mqa_dtype dt,
                                        int split_chunk);

/* Decode attention (as mqa_decode_attn) over a paged cache. */
mqa_status mqa_decode_attn_paged(const void *q, const void *k_pages,
                                 const void *v_pages, const int32_t *block_table,
                                 const int32_t *seq_lens, int b, int h, int g,
                                 int page_size, int max_pages, int num_pages,
                                 int d, mqa_dtype dt, float scale, float *out,
                                 void *workspace, size_t workspace_bytes,
                                 int split_chunk, int32_t *err_flags,
                                 hipStream_t stream);

/*
 * Several query tokens per sequence (T >= 1): a draft of T tokens verified in
 * one step, or a chunk of a prompt. [GQA notes] §八 (its reference code writes
 * the T new rows of the cache at once and attends them together) and §十
 * item 10 (the causal mask stays per query position when K/V heads are
 * shared).
 *
 *   q        : [b][T][h][d] of dt; token tau of sequence i sits at position
 *              seq_lens[i] - T + tau (seq_lens counts the T new tokens)
 *   k_new, v_new : [b][T][g][d] of dt; the append writes token tau to
 *              cache position seq_lens[i] - T + tau
 *   out      : [b][T][h][d] fp32; token tau attends positions
 *              t <= seq_lens[i] - T + tau (the causal mask)
 * A sequence with seq_lens[i] outside [T, S] is handled as an invalid length
 * (skipped by the append, NaN rows, MQA_DEVERR_SEQLEN). T must be in [1, S];
 * T = 1 is exactly mqa_append_kv / mqa_decode_attn (and the _paged calls).
 * For T > 1 the decode is bf16 only (MQA_F32: MQA_ERR_UNSUPPORTED) and runs
 * the matrix-core kernels. The workspace is
 * mqa_decode_multi_workspace_bytes() bytes, with S the capacity
 * (page_size * max_pages for a paged cache); the paged calls take their
 * arguments as in the paged section above.
 */
mqa_status mqa_append_kv_multi(void *k_cache, void *v_cache, const void *k_new,
                               const void *v_new, const int32_t *seq_lens,
                               int b, int T, int g, int S, int d, mqa_dtype dt,
                               int32_t *err_flags, hipStream_t stream);

size_t mqa_decode_multi_workspace_bytes(int b, int T, int h, int g, int S, int d,
                                        mqa_dtype dt, int split_chunk);

/* The schedule (mqa_schedule) a T-token call runs; -1: invalid arguments. */
int mqa_decode_multi_schedule(int b, int T, int h, int g, int S, int d,
                              mqa_dtype dt, int split_chunk);

mqa_status mqa_decode_attn_multi(const void *q, const void *k_cache,
                                 const void *v_cache, const int32_t *seq_lens,
                                 int b, int T, int h, int g, int S, int d,
                                 mqa_dtype dt, float scale, float *out,
                                 void *workspace, size_t workspace_bytes,
                                 int split_chunk, int32_t *err_flags,
                                 hipStream_t stream);

mqa_status mqa_append_kv_paged_multi(void *k_pages, void *v_pages,
                                     const void *k_new, const void *v_new,
                                     const int32_t *block_table,
                                     const int32_t *seq_lens, int b, int T,
                                     int g, int page_size, int max_pages,
                                     int num_pages, int d, mqa_dtype dt,
                                     int32_t *err_flags, hipStream_t stream);

mqa_status mqa_decode_attn_paged_multi(const void *q, const void *k_pages,
                                       const void *v_pages,
                                       const int32_t *block_table,
                                       const int32_t *seq_lens, int b, int T,
                                       int h, int g, int page_size,
                                       int max_pages, int num_pages, int d,
                                       mqa_dtype dt, float scale, float *out,
                                       void *workspace, size_t workspace_bytes,
                                       int split_chunk, int32_t *err_flags,
                                       hipStream_t stream);

/*
 * Low-precision cache: fp8 e4m3 codes with per-K/V-head scales. [GQA notes]
 * §十 item 7 (a quantised KV cache stacks with grouping but is validated on
 * its own); the pages fix no format, so: OCP E4M3FN codes (sign, 4 exponent
 * bits with bias 7, 3 mantissa bits, no infinity, S.1111.111 NaN, largest
 * finite 448), one fp32 scale per K/V head for K (k_scale[g]) and one for V
 * (v_scale[g]), device pointers; a cached value is code * scale[j]. The K/V
 * bytes per position halve against bf16.
 *
 *   k_cache, v_cache : [b][g][S][d] uint8 codes (pages: [num_pages][g][P][d])
 *   q                : [b][T][h][d] bf16 (T query tokens, T = 1: [b][h][d])
 *   k_new, v_new     : [b][T][g][d] bf16
 *   out              : [b][T][h][d] fp32
 * Append stores e4m3(x / scale[j]) for each new element: one correctly
 * rounded fp32 division, then the nearest code, ties to the even code,
 * magnitudes at or above 448 saturated (finite inputs never become NaN).
 * Decode computes the attention of the T-token section over the dequantised
 * values (codes are decoded exactly to bf16 for the matrix cores; the K scale
 * multiplies the scores, the V scale the outputs). Lengths, pages, the
 * workspace (mqa_decode_multi_workspace_bytes with dt = MQA_BF16) and the
 * errors are as above; the scale pointers must be 4-byte aligned.
 */
mqa_status mqa_append_kv_fp8(void *k_cache, void *v_cache, const void *k_new,
                             const void *v_new, const float *k_scale,
                             const float *v_scale, const int32_t *seq_lens,
                             int b, int T, int g, int S, int d,
                             int32_t *err_flags, hipStream_t stream);

mqa_status mqa_append_kv_paged_fp8(void *k_pages, void *v_pages,
                                   const void *k_new, const void *v_new,
                                   const float *k_scale, const float *v_scale,
                                   const int32_t *block_table,
                                   const int32_t *seq_lens, int b, int T, int g,
                                   int page_size, int max_pages, int num_pages,
                                   int d, int32_t *err_flags, hipStream_t stream);

mqa_status mqa_decode_attn_fp8(const void *q, const void *k_cache,
                               const void *v_cache, const float *k_scale,
                               const float *v_scale, const int32_t *seq_lens,
                               int b, int T, int h, int g, int S, int d,
                               float scale, float *out, void *workspace,
                               size_t workspace_bytes, int split_chunk,
                               int32_t *err_flags, hipStream_t stream);

mqa_status mqa_decode_attn_paged_fp8(const void *q, const void *k_pages,
                                     const void *v_pages, const float *k_scale,
                                     const float *v_scale,
                                     const int32_t *block_table,
                                     const int32_t *seq_lens, int b, int T,
                                     int h, int g, int page_size, int max_pages,
                                     int num_pages, int d, float scale,
                                     float *out, void *workspace,
                                     size_t workspace_bytes, int split_chunk,
                                     int32_t *err_flags, hipStream_t stream);

/*
 * int8 cache: the same layout, scales and calls' semantics as the fp8 cache
 * above, with two's-complement int8 codes ([MQA concept]'s risk list and
 * [MQA blog] §4.3 problem 3 speak of INT8 K/V; the pages fix no format):
 * a cached value is code * scale[j]. Append stores the nearest integer to
 * x / scale[j] (one correctly rounded fp32 division), ties to even,
 * saturated at +-127 (-128 is never written); NaN becomes 0. Decode goes
 * through mqa_decode_attn_ex with kv_dtype = MQA_INT8 (codes decoded
 * exactly to bf16; the K scale on the scores, the V scale on the outputs).
 *
 *   k_cache, v_cache : [b][g][S][d] int8 codes (pages: [num_pages][g][P][d])
 *   k_new, v_new     : [b][T][g][d] bf16
 */
mqa_status mqa_append_kv_int8(void *k_cache, void *v_cache, const void *k_new,
                              const void *v_new, const float *k_scale,
                              const float *v_scale, const int32_t *seq_lens,
                              int b, int T, int g, int S, int d,
                              int32_t *err_flags, hipStream_t stream);

mqa_status mqa_append_kv_paged_int8(void *k_pages, void *v_pages,
                                    const void *k_new, const void *v_new,
                                    const float *k_scale, const float *v_scale,
                                    const int32_t *block_table,
                                    const int32_t *seq_lens, int b, int T,
                                    int g, int page_size, int max_pages,
                                    int num_pages, int d, int32_t *err_flags,
                                    hipStream_t stream);

/*
 * One call with every option: layout (contiguous or paged), cache element
 * type (bf16, fp8 or int8 codes with scales, or f32), T query tokens, and a sliding window
 * ([MQA concept] 玩家對比 lists GQA with a sliding window: a query at position
 * p then sees only the positions t in (p - window, p]; the window start
 * replaces 0). The entry points above are this call with some fields fixed.
 * Fields not used by the chosen layout or type are ignored. f32 caches take
 * the one-token contiguous path only (T = 1, no window, no pages).
 */
typedef struct {
    const void *q;                  /* [b][T][h][d]: bf16 (f32 with an f32 cache) */
    const void *k, *v;              /* [b][g][S][d] or pages [num_pages][g][page_size][d] */
    const int32_t *block_table;     /* [b][max_pages] int32; NULL: contiguous cache */
    const int32_t *seq_lens;        /* [b], post-append lengths */
    const float *k_scale, *v_scale; /* [g] fp32, fp8 and int8 caches only */
    float *out;                     /* [b][T][h][d] fp32 */
    void *workspace;                /* mqa_decode_ex_workspace_bytes() bytes, 16-byte aligned */
    size_t workspace_bytes;
    int32_t *err_flags;             /* device int32 or NULL */
    int b, T, h, g, d;
    int S;                          /* contiguous capacity */
    int page_size, max_pages, num_pages;
    int kv_dtype;                   /* mqa_dtype of the cache */
    int window;                     /* > 0: sliding window of that many positions; 0: none */
    int split_chunk;                /* 0: automatic */
    float scale;                    /* softmax scale, normally 1/sqrt(d) */
} mqa_decode_desc;

/*
 * Workspace bytes mqa_decode_attn_ex needs for this descriptor; 0 when the
 * shape fields are invalid. Reads only the sizes, kv_dtype, window,
 * split_chunk and whether block_table is NULL: the data pointers may be
 * unset. mqa_decode_attn_ex checks the pointers (NULL: MQA_ERR_NULL; q, k,
 * v, out 16-byte aligned, scales 4-byte aligned: else MQA_ERR_ALIGN) and
 * that workspace_bytes is at least this figure (else MQA_ERR_WORKSPACE).
 */
size_t mqa_decode_ex_workspace_bytes(const mqa_decode_desc *desc);
mqa_status mqa_decode_attn_ex(const mqa_decode_desc *desc, hipStream_t stream);

/*
 * Rotary position embedding on bf16 rows. [GQA notes] §十 item 6: position
 * information is applied per head, to every query head and to each K/V
 * head's keys (shared or not); the pages give no formula, so the common
 * rotary form: pairs (x_i, x_{i+d/2}), i < d/2, are turned by the angle of
 * their position, a' = a c - b s, b' = b c + a s with (c, s) =
 * cos_sin[pos][i] (a caller-built fp32 table [n_pos][d/2][2], e.g. from
 * angles pos * base^(-2i/d)); each product and sum is rounded to fp32 in
 * that order (no fused multiply-add) and the results to bf16 (nearest,
 * ties to even). A position at or past n_pos is skipped and flagged
 * MQA_DEVERR_ROPE.
 *
 * mqa_rope_q rotates q [b][T][h][d] in place, token tau of sequence i at
 * position seq_lens[i] - T + tau. mqa_append_kv_rope is mqa_append_kv_multi
 * with each key row rotated at its position before it is stored (values as
 * they are); bf16 contiguous cache.
 */
mqa_status mqa_rope_q(void *q, const float *cos_sin, int n_pos, const int32_t *seq_lens, int b,
                      int T, int h, int d, int32_t *err_flags, hipStream_t stream);
mqa_status mqa_append_kv_rope(void *k_cache, void *v_cache, const void *k_new,
                              const void *v_new, const float *cos_sin, int n_pos,
                              const int32_t *seq_lens, int b, int T, int g, int S, int d,
                              int32_t *err_flags, hipStream_t stream);

/* Static text for a status code (never NULL). */
const char *mqa_status_string(mqa_status s);

/*
 * KV-cache bytes of `layers` layers, [GQA notes] §一/§七 and [MQA concept]
 * 技術原理: 2 * layers * g * S * d * dtype_bytes (the factor 2 is K and V).
 */
uint64_t mqa_kv_bytes(int layers, int g, int64_t S, int d, int dtype_bytes);

#ifdef __cplusplus
}
#endif
#endif /* MQA_DECODE_H */

// libmqa_decode: decode attention over a shared-head KV cache on gfx950.
//
// One decode step ([GQA notes] = ybb.press "分组查询注意力（GQA）与多查询注意力
// （MQA）深度实战"): append the new token's K/V to the cache (§八; nanhubrain.csdn.net
// MQA article §2.2), then for every query head hq of every sequence i, with
// G = h/g query heads per K/V head and j = hq / G (§五),
//   out[i,hq,:] = softmax_t(scale * q[i,hq,:] . K[i,j,t,:]) V[i,j,t,:],  t < L_i.
//
// Kernels, in the order of this file
//   append_kv_kernel, append_kv_paged_kernel
//                        the step's new K/V rows into a contiguous or paged
//                        bf16/fp32 cache: one 16-byte chunk per thread, bit copy.
//   append_kv_codes_kernel
//                        the same into a one-byte cache: each value divided by
//                        its K/V head's scale and rounded to an e4m3 or int8 code.
//   rope_q_kernel, append_kv_rope_kernel
//                        rotary position embedding of the query rows in place,
//                        and of the keys on their way into the cache.
//   split_rows_kernel    vector-ALU decode (fp32 caches, and bf16 when the caller
//                        asks for it): one work-group per (partition, K/V head,
//                        block of query heads, sequence); 64-row K/V tiles go
//                        global->LDS by DMA and serve every query head of the
//                        group; one lane per cache row for the scores, one
//                        16-byte column chunk per lane for P.V.
//   split_mfma_kernel    matrix-core decode over fixed partitions (bf16 or
//                        one-byte caches): scores as K.Q^T and P.V with
//                        v_mfma_f32_16x16x32_bf16, 32 cache rows per step, the
//                        unit's query rows in blocks of 16, online softmax in
//                        the accumulator layout; writes per-partition partials.
//   split_pair_kernel    the same for units of more than 16 query rows: pairs of
//                        waves share each loaded step through LDS.
//   streamk_mfma_kernel  the balanced schedule (many ragged units): one
//                        work-group per compute unit takes an equal share of all
//                        units' steps, its waves claiming steps from an LDS
//                        counter; writes out directly, and partials only for
//                        the units cut between two shares.
//   streamk_combine_kernel
//                        merges the pieces of those cut units into out.
//   combine_kernel       log-sum-exp merge of the fixed partitions into out.
// Decode runs split_rows_kernel or split_mfma/split_pair_kernel followed by
// combine_kernel, or streamk_mfma_kernel followed by streamk_combine_kernel;
// which one is decided on the host from the shapes (use_streamk below).
//
// Everything is enqueued on the caller's stream; nothing is allocated here.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <tuple>
#include <type_traits>
#include <utility>

#include "mqa_decode.h"

namespace {

constexpr int kTile = 64;  // cache rows per tile (one per lane in the score phase)

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// c + a.lo*b.lo + a.hi*b.hi for two packed bfloat16 pairs, fp32 accumulate.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Reductions over the 64 lanes of a wave: DPP within each row of 16 lanes
// (xor 1, xor 2, half-row mirror, row mirror), then two cross-row exchanges.
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_f32<0xB1>(x));   // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp_f32<0x4E>(x));   // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp_f32<0x141>(x));  // row_half_mirror
    x = fmaxf(x, dpp_f32<0x140>(x));  // row_mirror
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_f32<0xB1>(x);
    x += dpp_f32<0x4E>(x);
    x += dpp_f32<0x141>(x);
    x += dpp_f32<0x140>(x);
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));  // 16 bytes
// Raw buffer descriptor over [base, base + bytes): offsets are 32-bit, the
// base sits in scalar registers, and a load whose offset is at or past
// `bytes` returns zeros without a memory access. Word 3 is the raw-buffer
// format of the gfx9 family.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;  // wave-uniform by construction
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), (short)0,
                                             (int)bytes, 0x00020000);
}
// 16 bytes through a descriptor, non-temporal (streamed once)
__device__ __forceinline__ u32x4_t buffer_stream16(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}
// 16 bytes through a descriptor, cached (read again soon by another wave)
__device__ __forceinline__ u32x4_t buffer_cached16(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// 16-byte global -> LDS copy. The LDS destination of lane l is
// lds_block + 16*l (lds_block is wave-uniform and goes through m0, which is
// saved and restored around the copy; one wait state separates the m0 write
// from the instruction that reads it). The instruction has no register
// result; completion is awaited explicitly with vmem_wait_barrier() before
// the LDS block is read. Written as asm because the compiler, seeing the
// builtin form, waits for every pending copy before any LDS read and so
// serialises the prefetch of the next tile with the work on this one.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_block) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_block), "v"(src)
        : "memory");
}

// Wait until at most N vector-memory operations of this wave are pending and
// its LDS accesses are done, then work-group barrier.
template <int N>
__device__ __forceinline__ void vmem_wait_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

// Work-group barrier after this wave's LDS accesses have completed.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const lds_u8 *)p;
}

// ---------------------------------------------------------------------------
// append
// ---------------------------------------------------------------------------

// Where thread t of an append works: one 16-byte chunk c of token tau of
// K/V head j of sequence i, in tensor `which` (0: K, 1: V).
struct AppendSlot {
    int c, j, tau, i, which;
    __device__ AppendSlot(long long t, int cpr, int b, int T, int g) {
        c = (int)(t % cpr);
        t /= cpr;
        j = (int)(t % g);
        t /= g;
        tau = (int)(t % T);
        t /= T;
        i = (int)(t % b);
        which = (int)(t / b);
    }
    __device__ bool first() const { return c == 0 && j == 0 && tau == 0 && which == 0; }
};

// Token tau of the step's T (k_new/v_new [b][T][g][d]) goes to position
// L - T + tau of its K/V head ([MQA blog] §2.2; [GQA notes] §八 writes the T
// rows at once); lengths outside [T, S] are skipped and flagged.
__global__ void append_kv_kernel(uint8_t *__restrict__ kc, uint8_t *__restrict__ vc,
                                 const uint8_t *__restrict__ kn, const uint8_t *__restrict__ vn,
                                 const int32_t *__restrict__ seq_lens, int b, int T, int g, int S,
                                 int row_bytes, int32_t *__restrict__ err) {
    const int cpr = row_bytes >> 4;
    const long long total = 2ll * b * T * g * cpr;
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= total) return;
    const AppendSlot a(t, cpr, b, T, g);
    const int L = seq_lens[a.i];
    if (L < T || L > S) {
        if (a.first() && err) atomicOr(err, MQA_DEVERR_SEQLEN);
        return;
    }
    const size_t src = (((size_t)a.i * T + a.tau) * g + a.j) * row_bytes + (size_t)a.c * 16;
    const size_t dst = (((size_t)a.i * g + a.j) * S + (size_t)(L - T + a.tau)) * row_bytes +
                       (size_t)a.c * 16;
    const uint8_t *s = a.which ? vn : kn;
    uint8_t *dp = a.which ? vc : kc;
    *(uint4 *)(dp + dst) = *(const uint4 *)(s + src);
}

// Paged cache: position p = L - T + tau goes to row p % P of page
// block_table[i][p / P] of pages [num_pages][g][P][d]. A page id outside
// [0, num_pages) is skipped and flagged.
__global__ void append_kv_paged_kernel(uint8_t *__restrict__ kp, uint8_t *__restrict__ vp,
                                       const uint8_t *__restrict__ kn, const uint8_t *__restrict__ vn,
                                       const int32_t *__restrict__ block_table,
                                       const int32_t *__restrict__ seq_lens, int b, int T, int g,
                                       int P, int max_pages, int num_pages, int row_bytes,
                                       int32_t *__restrict__ err) {
    const int cpr = row_bytes >> 4;
    const long long total = 2ll * b * T * g * cpr;
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= total) return;
    const AppendSlot a(t, cpr, b, T, g);
    const int L = seq_lens[a.i];
    if (L < T || L > P * max_pages) {
        if (a.first() && err) atomicOr(err, MQA_DEVERR_SEQLEN);
        return;
    }
    const int pos = L - T + a.tau;
    const int page = block_table[(size_t)a.i * max_pages + pos / P];
    if (page < 0 || page >= num_pages) {
        if (a.c == 0 && a.j == 0 && a.which == 0 && err) atomicOr(err, MQA_DEVERR_PAGE);
        return;
    }
    const size_t src = (((size_t)a.i * T + a.tau) * g + a.j) * row_bytes + (size_t)a.c * 16;
    const size_t dst = (((size_t)page * g + a.j) * P + (size_t)(pos % P)) * row_bytes + (size_t)a.c * 16;
    const uint8_t *s = a.which ? vn : kn;
    uint8_t *dp = a.which ? vp : kp;
    *(uint4 *)(dp + dst) = *(const uint4 *)(s + src);
}

// fp8 e4m3 (OCP E4M3FN: bias 7, 3 mantissa bits, no infinity, largest
// finite 448) code of f: the nearest value, ties to the even code;
// magnitudes at or above 448 saturate to +-448, so a finite value never
// becomes NaN; NaN stays NaN.
__device__ __forceinline__ uint32_t e4m3_code(float f) {
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return sign | 0x7fu;   // NaN
    if (a >= 0x43e00000u) return sign | 0x7eu;  // >= 448, infinity included
    if (a < 0x3c800000u)                        // below 2^-6: multiples of 2^-9 (code 8 = 2^-6)
        return sign | (uint32_t)__builtin_rintf(__builtin_bit_cast(float, a) * 512.0f);
    // normal: exponent re-biased (127 -> 7), 3 of 23 mantissa bits kept,
    // nearest-even on the 20 dropped (a carry moves to the next exponent)
    uint32_t code = (((a >> 23) - 120u) << 3) | ((a >> 20) & 7u);
    const uint32_t rem = a & 0xfffffu;
    if (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) code += 1;
    return sign | code;
}

// int8 code (two's complement, in the low byte) of f: the nearest integer,
// ties to even, saturated at +-127 (-128 is never produced); NaN becomes 0.
__device__ __forceinline__ uint32_t int8_code(float f) {
    if (f != f) return 0u;
    const float r = fminf(fmaxf(__builtin_rintf(f), -127.f), 127.f);
    return (uint32_t)(int)r & 0xffu;
}

// Quantised append into a one-byte cache: token tau of the new rows (bf16
// [b][T][g][d]) goes to position L - T + tau as code(x / scale[j]), one
// correctly rounded fp32 division per element ([GQA notes] §十 item 7: a
// quantised KV cache); the code is e4m3 or, with I8, int8. Contiguous cache
// [b][g][S][d] (bt NULL) or pages [num_pages][g][P][d] through block table
// bt (S then the page size P). Thread t converts one 8-element chunk.
template <bool I8>
__global__ void append_kv_codes_kernel(uint8_t *__restrict__ kc, uint8_t *__restrict__ vc,
                                     const uint16_t *__restrict__ kn,
                                     const uint16_t *__restrict__ vn,
                                     const float *__restrict__ k_scale,
                                     const float *__restrict__ v_scale,
                                     const int32_t *__restrict__ bt,
                                     const int32_t *__restrict__ seq_lens, int b, int T, int g,
                                     int S, int max_pages, int num_pages, int d,
                                     int32_t *__restrict__ err) {
    const int cpr = d >> 3;
    const long long total = 2ll * b * T * g * cpr;
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= total) return;
    const AppendSlot a(t, cpr, b, T, g);
    const int L = seq_lens[a.i];
    const int cap = bt ? S * max_pages : S;
    if (L < T || L > cap) {
        if (a.first() && err) atomicOr(err, MQA_DEVERR_SEQLEN);
        return;
    }
    const int pos = L - T + a.tau;
    size_t row;
    if (bt) {
        const int page = bt[(size_t)a.i * max_pages + pos / S];
        if (page < 0 || page >= num_pages) {
            if (a.c == 0 && a.j == 0 && a.which == 0 && err) atomicOr(err, MQA_DEVERR_PAGE);
            return;
        }
        row = ((size_t)page * g + a.j) * S + pos % S;
    } else {
        row = ((size_t)a.i * g + a.j) * S + pos;
    }
    const uint16_t *src = (a.which ? vn : kn) + (((size_t)a.i * T + a.tau) * g + a.j) * d + 8 * a.c;
    const float sc = (a.which ? v_scale : k_scale)[a.j];
    const u32x4_t in = *(const u32x4_t *)src;  // 8 bf16
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 8; e++) {
        const uint32_t bits = (in[e >> 1] >> (16 * (e & 1))) << 16;  // bf16 -> fp32, exact
        const float y = __fdiv_rn(__builtin_bit_cast(float, bits), sc);
        const uint32_t code = I8 ? int8_code(y) : e4m3_code(y);
        if (e < 4)
            lo |= code << (8 * e);
        else
            hi |= code << (8 * (e - 4));
    }
    *(uint2 *)((a.which ? vc : kc) + row * d + 8 * a.c) = make_uint2(lo, hi);
}

// ---------------------------------------------------------------------------
// rotary position embedding on bf16 rows
// ---------------------------------------------------------------------------

// Nearest bf16 of a float, ties to even (NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Rotate 8 pairs of a bf16 row in place: elements i0 .. i0+7 (a) and their
// partners i0 + d/2 .. (b), turned by the angles of position pos: a' = a c -
// b s, b' = b c + a s, each product and sum rounded to fp32 in that order
// (no fused multiply-add), then to bf16 ([GQA notes] §十 item 6: position
// information applied per head, to queries and keys alike; cos_sin [n][d/2][2]).
__device__ __forceinline__ void rope8(const u32x4_t &a_in, const u32x4_t &b_in, const float *cs,
                                      u32x4_t &a_out, u32x4_t &b_out) {
#pragma clang fp contract(off)  // each product rounded on its own, as specified
#pragma unroll
    for (int w = 0; w < 4; w++) {
        uint32_t ra = 0, rb = 0;
#pragma unroll
        for (int hlf = 0; hlf < 2; hlf++) {
            const int e = 2 * w + hlf;
            const float a = __builtin_bit_cast(float, (a_in[w] >> (16 * hlf)) << 16);
            const float b = __builtin_bit_cast(float, (b_in[w] >> (16 * hlf)) << 16);
            const float c = cs[2 * e], sn = cs[2 * e + 1];
            const float ac = a * c, bs = b * sn, bc = b * c, as = a * sn;
            const float na = ac - bs, nb = bc + as;
            ra |= bf16_rne(na) << (16 * hlf);
            rb |= bf16_rne(nb) << (16 * hlf);
        }
        a_out[w] = ra;
        b_out[w] = rb;
    }
}

// q [b][T][h][d] rotated in place, token tau of sequence i at position
// L_i - T + tau. Thread t takes 8 pairs of one row.
__global__ void rope_q_kernel(uint16_t *__restrict__ q, const float *__restrict__ cos_sin, int n_pos,
                              const int32_t *__restrict__ seq_lens, int b, int T, int h, int d,
                              int32_t *__restrict__ err) {
    const int groups = d >> 4;  // 8-pair groups per row
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (long long)b * T * h * groups) return;
    const int c = (int)(t % groups);
    const long long row = t / groups;  // (i, tau, hq)
    const int tau = (int)(row / h % T), i = (int)(row / h / T);
    const int pos = seq_lens[i] - T + tau;
    if (pos < 0 || pos >= n_pos) {
        if (c == 0 && row % h == 0 && err) atomicOr(err, pos < 0 ? MQA_DEVERR_SEQLEN : MQA_DEVERR_ROPE);
        return;
    }
    uint16_t *x = q + row * d + 8 * c;
    const float *cs = cos_sin + ((size_t)pos * (d >> 1) + 8 * c) * 2;
    u32x4_t a = *(const u32x4_t *)x, bb = *(const u32x4_t *)(x + (d >> 1));
    u32x4_t na, nb;
    rope8(a, bb, cs, na, nb);
    *(u32x4_t *)x = na;
    *(u32x4_t *)(x + (d >> 1)) = nb;
}

// The T-token append with the keys rotated at their positions (values as
// they are): bf16 cache [b][g][S][d], new rows [b][T][g][d]. Thread t takes
// 8 pairs of one (sequence, token, K/V head).
__global__ void append_kv_rope_kernel(uint16_t *__restrict__ kc, uint16_t *__restrict__ vc,
                                      const uint16_t *__restrict__ kn,
                                      const uint16_t *__restrict__ vn,
                                      const float *__restrict__ cos_sin, int n_pos,
                                      const int32_t *__restrict__ seq_lens, int b, int T, int g,
                                      int S, int d, int32_t *__restrict__ err) {
    const int groups = d >> 4;
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (long long)b * T * g * groups) return;
    const int c = (int)(t % groups);
    const long long r = t / groups;  // ((i * T + tau) * g + j)
    const int j = (int)(r % g), tau = (int)(r / g % T), i = (int)(r / g / T);
    const bool first = c == 0 && j == 0 && tau == 0;
    const int L = seq_lens[i];
    if (L < T || L > S) {
        if (first && err) atomicOr(err, MQA_DEVERR_SEQLEN);
        return;
    }
    const int pos = L - T + tau;
    if (pos >= n_pos) {
        if (c == 0 && j == 0 && err) atomicOr(err, MQA_DEVERR_ROPE);
        return;
    }
    const size_t src = (size_t)r * d + 8 * c;
    const size_t dst = (((size_t)i * g + j) * S + pos) * d + 8 * c;
    const int hd = d >> 1;
    u32x4_t na, nb;
    rope8(*(const u32x4_t *)(kn + src), *(const u32x4_t *)(kn + src + hd),
          cos_sin + ((size_t)pos * hd + 8 * c) * 2, na, nb);
    *(u32x4_t *)(kc + dst) = na;
    *(u32x4_t *)(kc + dst + hd) = nb;
    *(u32x4_t *)(vc + dst) = *(const u32x4_t *)(vn + src);
    *(u32x4_t *)(vc + dst + hd) = *(const u32x4_t *)(vn + src + hd);
}

// ---------------------------------------------------------------------------
// split kernel: one wave per query head in the score phase, one lane per row
// ---------------------------------------------------------------------------

template <typename T, int D, int HPW>
struct RowsCfg {
    static constexpr int EB = (int)sizeof(T);
    static constexpr int ROW_BYTES = D * EB;          // 128 .. 512
    static constexpr int CPR = ROW_BYTES / 16;        // 16-byte chunks per row
    static constexpr int NW = HPW;                    // waves per work-group
    static constexpr int NT = 64 * NW;
    static constexpr int TILE_BYTES = kTile * ROW_BYTES;
    static constexpr int DMA = TILE_BYTES / 16 / NT;  // DMA loads per lane per K (or V) tile
    static constexpr int ROW_DW = ROW_BYTES / 4;
    // P.V phase: each lane owns a VCB-byte column chunk of some rows; 8-byte
    // chunks keep the 8 heads' accumulators of the bf16 case at 32 registers.
    static constexpr int VCB = (EB == 2 && HPW == 8) ? 8 : 16;
    static constexpr int ELEMS = VCB / EB;            // columns per lane
    static constexpr int CPRV = ROW_BYTES / VCB;      // column chunks per row
    static constexpr int RPW = kTile / NW;            // rows per wave in the P.V phase
    static constexpr int RPI = 64 / CPRV;             // rows covered by one wave-wide read
    static constexpr int VROWS = RPW / RPI;           // rows per lane in the P.V phase
    // two 8-wave work-groups per compute unit need <= 128 registers per lane
    static constexpr int WAVES_PER_EU = (HPW == 8 && ROW_BYTES <= 256) ? 4 : 1;
    static_assert(DMA >= 1 && VROWS >= 1, "too many waves for this row size");
    static_assert(NW * HPW * D * 4 <= 2 * 2 * TILE_BYTES, "reduction scratch must fit");
};

template <typename T, int D, int HPW>
struct RowsSmem {
    using C = RowsCfg<T, D, HPW>;
    uint8_t kv[2][2][C::TILE_BYTES];  // [stage][K=0, V=1], rows XOR-swizzled by 16-byte chunk
    float p[2][kTile][HPW];           // softmax numerators of a tile, [row][head]
    float alpha[2][HPW];              // rescale factor of the running sums, per head
};

// Scores more than 2^kSlack above the reference max of a head trigger a
// rescale of its running sums; below that the reference is kept, so the
// exponentials stay <= 2^kSlack and most tiles skip the rescale entirely.
constexpr float kSlack = 8.0f;

// Tile DMA: row r, chunk c of a 64-row tile lands at LDS offset
// r*ROW_BYTES + 16*(c ^ (r % CPR)), so that a 64-lane read of one chunk of 64
// rows, or of 64 chunks of 4 rows, touches 64 distinct 16-byte bank groups.
// Lane `lane` of wave `w` copies, in its r-th instruction, the chunk whose
// byte offset from the tile's first row is dma_off(w, lane, r).
template <typename C>
__device__ __forceinline__ int dma_row(int w, int lane, int r) {
    return ((w * C::DMA + r) * 64 + lane) / C::CPR;
}
template <typename C>
__device__ __forceinline__ uint32_t dma_off(int w, int lane, int r) {
    const int slot = (w * C::DMA + r) * 64 + lane;
    const int row = slot / C::CPR;
    return (uint32_t)(row * C::ROW_BYTES + (((slot % C::CPR) ^ (row % C::CPR)) << 4));
}

// 16-byte global -> LDS copy from a wave-uniform base plus a per-lane 32-bit
// byte offset (same m0 handling as dma16).
__device__ __forceinline__ void dma16_sv(const void *sbase, uint32_t voff, uint32_t lds_block) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_block), "v"(voff), "s"(sbase)
        : "memory");
}

template <typename C, bool TAIL>
__device__ __forceinline__ void dma_tile(const uint8_t *__restrict__ base, int t0, int S,
                                         uint32_t lds_tile, const uint32_t (&off)[C::DMA], int w,
                                         int lane) {
    if constexpr (!TAIL) {
        const uint8_t *tile = base + (size_t)t0 * C::ROW_BYTES;
#pragma unroll
        for (int r = 0; r < C::DMA; r++)
            dma16_sv(tile, off[r], lds_tile + (w * C::DMA + r) * 1024);
    } else {
        // rows past the capacity are clamped to the last row (never used)
#pragma unroll
        for (int r = 0; r < C::DMA; r++) {
            const int row = dma_row<C>(w, lane, r);
            const int grow = min(t0 + row, S - 1);
            const uint32_t col = off[r] - (uint32_t)(row * C::ROW_BYTES);
            dma16(base + (size_t)grow * C::ROW_BYTES + col, lds_tile + (w * C::DMA + r) * 1024);
        }
    }
}

template <bool V> struct TailTag { static constexpr bool value = V; };

template <typename T, int D, int HPW>
__global__ void __launch_bounds__(64 * HPW)
__attribute__((amdgpu_waves_per_eu(RowsCfg<T, D, HPW>::WAVES_PER_EU, 8)))
split_rows_kernel(const T *__restrict__ q, const T *__restrict__ kc, const T *__restrict__ vc,
                  const int32_t *__restrict__ seq_lens, int h, int g, int S, int G, int nhc,
                  int chunk, int nsplit, float qk_scale_log2, float *__restrict__ part_o,
                  float2 *__restrict__ part_ml) {
    using C = RowsCfg<T, D, HPW>;
    __shared__ __attribute__((aligned(1024))) RowsSmem<T, D, HPW> sm;

    const int s = blockIdx.x;
    const int j = blockIdx.y / nhc;
    const int hc = blockIdx.y % nhc;
    const int i = blockIdx.z;
    const int L = seq_lens[i];
    if (L < 1 || L > S) return;  // reported by the combine
    const int t_begin = s * chunk;
    if (t_begin >= L) return;  // partition past this sequence's length
    const int t_end = min(t_begin + chunk, L);
    const int ntiles = (t_end - t_begin + kTile - 1) / kTile;

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    const size_t head_row0 = ((size_t)i * g + j) * (size_t)S;
    const uint8_t *kbase = (const uint8_t *)kc + head_row0 * C::ROW_BYTES;
    const uint8_t *vbase = (const uint8_t *)vc + head_row0 * C::ROW_BYTES;

    // Query head scored by this wave (slots past G repeat the last head and
    // are never written out). Its row stays in scalar registers.
    const int slot_w = hc * HPW + w;
    const int hq_w = j * G + min(slot_w, G - 1);
    const uint32_t *qrow = (const uint32_t *)(q + ((size_t)i * h + hq_w) * D);
    uint32_t qv[C::ROW_DW];
#pragma unroll
    for (int x = 0; x < C::ROW_DW; x++) qv[x] = qrow[x];

    // per-lane constant offsets
    uint32_t doff[C::DMA];
#pragma unroll
    for (int r = 0; r < C::DMA; r++) doff[r] = dma_off<C>(w, lane, r);
    const uint32_t smem = lds_addr(&sm);
    const uint32_t kv_base = lds_addr(&sm.kv[0][0][0]);
    // score phase: lane reads row `lane`, chunk c at koff ^ (c << 4)
    const uint32_t koff = (uint32_t)(lane * C::ROW_BYTES + ((lane % C::CPR) << 4));
    // P.V phase: lane -> (row group rg, VCB-byte column chunk cc)
    const int rg = lane / C::CPRV;
    const int cc = lane % C::CPRV;
    constexpr int SUB = 16 / C::VCB;  // column chunks per 16-byte granule
    uint32_t voff[C::VROWS];
    int vrow[C::VROWS];
#pragma unroll
    for (int r = 0; r < C::VROWS; r++) {
        vrow[r] = w * C::RPW + r * C::RPI + rg;
        voff[r] = (uint32_t)(vrow[r] * C::ROW_BYTES + (((cc / SUB) ^ (vrow[r] % C::CPR)) << 4) +
                             (cc % SUB) * C::VCB);
    }

    float acc[HPW][C::ELEMS];
#pragma unroll
    for (int a = 0; a < HPW; a++)
#pragma unroll
        for (int e = 0; e < C::ELEMS; e++) acc[a][e] = 0.f;
    float m_ref = -INFINITY;  // reference max of this wave's head (log2 units)
    float l_lane = 0.f;       // this lane's share of the running sum

    auto stage_k = [&](int st) { return kv_base + (uint32_t)((2 * st) * C::TILE_BYTES); };
    auto stage_v = [&](int st) { return kv_base + (uint32_t)((2 * st + 1) * C::TILE_BYTES); };

    auto issue_k = [&](int n, int st) {
        const int t0 = t_begin + n * kTile;
        if (t0 + kTile <= S) dma_tile<C, false>(kbase, t0, S, stage_k(st), doff, w, lane);
        else dma_tile<C, true>(kbase, t0, S, stage_k(st), doff, w, lane);
    };
    auto issue_v = [&](int n, int st) {
        const int t0 = t_begin + n * kTile;
        if (t0 + kTile <= S) dma_tile<C, false>(vbase, t0, S, stage_v(st), doff, w, lane);
        else dma_tile<C, true>(vbase, t0, S, stage_v(st), doff, w, lane);
    };

    // Scores of tile n: lane = cache row, wave = query head; online-softmax
    // bookkeeping; the numerators go to pbuf[n & 1], the head's rescale
    // factor to alpha[n & 1]. TAIL masks rows >= t_end.
    auto scores = [&](int n, auto tail_tag) {
        constexpr bool TAIL = decltype(tail_tag)::value;
        const int t0 = t_begin + n * kTile;
        const uint8_t *lds = (const uint8_t *)&sm;
        const uint32_t kb = stage_k(n & 1) - smem + koff;
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
        for (int c = 0; c < C::CPR; c++) {
            const uint4 kk = *(const uint4 *)(lds + (kb ^ (uint32_t)(c << 4)));
            if constexpr (sizeof(T) == 2) {
                a0 = dot2_bf16(qv[4 * c + 0], kk.x, a0);
                a1 = dot2_bf16(qv[4 * c + 1], kk.y, a1);
                a2 = dot2_bf16(qv[4 * c + 2], kk.z, a2);
                a3 = dot2_bf16(qv[4 * c + 3], kk.w, a3);
            } else {
                a0 = fmaf(__uint_as_float(qv[4 * c + 0]), __uint_as_float(kk.x), a0);
                a1 = fmaf(__uint_as_float(qv[4 * c + 1]), __uint_as_float(kk.y), a1);
                a2 = fmaf(__uint_as_float(qv[4 * c + 2]), __uint_as_float(kk.z), a2);
                a3 = fmaf(__uint_as_float(qv[4 * c + 3]), __uint_as_float(kk.w), a3);
            }
        }
        float s2 = ((a0 + a1) + (a2 + a3)) * qk_scale_log2;
        if constexpr (TAIL) s2 = (t0 + lane < t_end) ? s2 : -INFINITY;
        float alpha = 1.f;
        // The cross-lane max is needed only when some score passes the
        // reference by more than the slack (always on the first tile).
        if (__any(s2 > m_ref + kSlack)) {  // wave-uniform
            const float mt = wave_max(s2);
            alpha = fast_exp2(m_ref - mt);
            m_ref = mt;
        }
        const float p = fast_exp2(s2 - m_ref);
        l_lane = fmaf(l_lane, alpha, p);
        sm.p[n & 1][lane][w] = p;
        if (lane == 0) sm.alpha[n & 1][w] = alpha;
    };

    // P.V of tile n: lane owns column chunk cc of rows vrow[0..VROWS).
    auto pv = [&](int n, auto tail_tag) {
        constexpr bool TAIL = decltype(tail_tag)::value;
        const int t0 = t_begin + n * kTile;
        const uint8_t *lds = (const uint8_t *)&sm;
        float al[HPW];
        bool rescale = false;
#pragma unroll
        for (int a = 0; a < HPW; a++) {
            al[a] = sm.alpha[n & 1][a];
            rescale |= al[a] != 1.f;
        }
        if (rescale) {  // uniform across the work-group
#pragma unroll
            for (int a = 0; a < HPW; a++)
#pragma unroll
                for (int e = 0; e < C::ELEMS; e++) acc[a][e] *= al[a];
        }
        const uint32_t vb = stage_v(n & 1) - smem;
#pragma unroll
        for (int r = 0; r < C::VROWS; r++) {
            float vf[C::ELEMS];
            if constexpr (C::VCB == 8) {
                const uint2 vv = *(const uint2 *)(lds + vb + voff[r]);
                vf[0] = bf16_lo(vv.x); vf[1] = bf16_hi(vv.x);
                vf[2] = bf16_lo(vv.y); vf[3] = bf16_hi(vv.y);
            } else if constexpr (sizeof(T) == 2) {
                const uint4 vv = *(const uint4 *)(lds + vb + voff[r]);
                vf[0] = bf16_lo(vv.x); vf[1] = bf16_hi(vv.x);
                vf[2] = bf16_lo(vv.y); vf[3] = bf16_hi(vv.y);
                vf[4] = bf16_lo(vv.z); vf[5] = bf16_hi(vv.z);
                vf[6] = bf16_lo(vv.w); vf[7] = bf16_hi(vv.w);
            } else {
                const uint4 vv = *(const uint4 *)(lds + vb + voff[r]);
                vf[0] = __uint_as_float(vv.x); vf[1] = __uint_as_float(vv.y);
                vf[2] = __uint_as_float(vv.z); vf[3] = __uint_as_float(vv.w);
            }
            if constexpr (TAIL) {
                // rows past the end may hold anything (even NaN): never let them in
                const bool ok = t0 + vrow[r] < t_end;
#pragma unroll
                for (int e = 0; e < C::ELEMS; e++) vf[e] = ok ? vf[e] : 0.f;
            }
            float pr[HPW];
#pragma unroll
            for (int a = 0; a < HPW; a++) pr[a] = sm.p[n & 1][vrow[r]][a];
#pragma unroll
            for (int a = 0; a < HPW; a++)
#pragma unroll
                for (int e = 0; e < C::ELEMS; e++) acc[a][e] = fmaf(pr[a], vf[e], acc[a][e]);
        }
    };

    // Software pipeline, one barrier per tile. Iteration n: wait for K(n) and
    // V(n-1) (everything issued in iteration n-1) and for every wave to have
    // finished iteration n-1; start copying K(n+1) and V(n); scores of tile n;
    // P.V of tile n-1. Stages are reused two iterations after their copy.
    const bool last_full = t_begin + ntiles * kTile <= t_end;
    issue_k(0, 0);
    for (int n = 0; n <= ntiles; n++) {
        vmem_wait_barrier<0>();
        if (n + 1 < ntiles) issue_k(n + 1, (n + 1) & 1);
        if (n < ntiles) {
            issue_v(n, n & 1);
            if (n + 1 < ntiles || last_full) scores(n, TailTag<false>{});
            else scores(n, TailTag<true>{});
        }
        if (n >= 1) {
            if (n < ntiles || last_full) pv(n - 1, TailTag<false>{});
            else pv(n - 1, TailTag<true>{});
        }
    }

    // ---- partition result: (m, l) per head, sum of acc over lanes and waves ----
    const float l_tot = wave_sum(l_lane);
#pragma unroll
    for (int a = 0; a < HPW; a++)
#pragma unroll
        for (int e = 0; e < C::ELEMS; e++) {
            float x = acc[a][e];
#pragma unroll
            for (int off = C::CPRV; off < 64; off <<= 1) x += __shfl_xor(x, off);
            acc[a][e] = x;
        }
    lds_barrier();  // every wave is done with the tiles; reuse them as scratch
    float *red = (float *)&sm.kv[0][0][0];  // [NW][HPW][D]
    if (lane < C::CPRV) {
#pragma unroll
        for (int a = 0; a < HPW; a++)
#pragma unroll
            for (int e = 0; e < C::ELEMS; e++) red[(w * HPW + a) * D + lane * C::ELEMS + e] = acc[a][e];
    }
    lds_barrier();
    for (int idx = threadIdx.x; idx < HPW * D; idx += C::NT) {
        const int a = idx / D, x = idx % D;
        if (hc * HPW + a >= G) continue;
        float sum = 0.f;
#pragma unroll
        for (int ww = 0; ww < C::NW; ww++) sum += red[(ww * HPW + a) * D + x];
        const size_t hq = (size_t)i * h + j * G + hc * HPW + a;
        part_o[(hq * nsplit + s) * D + x] = sum;
    }
    if (lane == 0 && slot_w < G) {
        const size_t hq = (size_t)i * h + j * G + slot_w;
        part_ml[hq * nsplit + s] = make_float2(m_ref, l_tot);
    }
}

// ---------------------------------------------------------------------------
// bf16 partition kernels: matrix cores for both contractions
// ---------------------------------------------------------------------------
//
// Per 32-position step of one wave, with 16 query heads of the group as the
// 16-wide matrix dimension (padded when fewer than 16):
//   S^T[pos][head] = K[pos][:] . Q[head][:]     two 16x16x32 bf16 MFMA blocks
//                                               per 32 d (fp32 accumulate;
//                                               bf16 products are exact)
//   O[head][x]    += P[head][pos] V[pos][x]     P split as bf16 hi + lo
//                                               (two MFMAs, ~2^-17 relative)
// Lane l (r = l % 16, qd = l / 16) holds S^T rows pos = 4qd+v (v < 4) of each
// 16-position block for head r: exactly the A-operand slots of P for the
// P.V MFMA if the 32 positions of a step are numbered
//   kslot(qd, e) = 4qd + e (e < 4),  16 + 4qd + (e - 4) (e >= 4),
// so P never moves. V needs a transposed read (8 positions of one column per
// lane); it goes through a small wave-private LDS buffer with padded rows.
// Each wave runs its own online softmax over its steps; the waves are merged
// through LDS at the end of a partition.

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

template <int D>
struct MfmaCfg {
    static constexpr int ROW_BYTES = D * 2;
    static constexpr int KSTEPS = D / 32;            // 32-wide d slices of the score MFMA
    static constexpr int NB = D / 16;                // 16-column blocks of the P.V MFMA
    static constexpr int STEP = 32;                  // positions per step
    static constexpr int NW = 4;                     // waves per work-group
    static constexpr int CPR = ROW_BYTES / 16;       // 16-byte chunks per row
    static constexpr int RPI = 64 / CPR;             // rows per wave-wide V load
    static constexpr int VLOADS = STEP / RPI;        // V loads per lane per step
    static constexpr int VSTRIDE = ROW_BYTES + 32;   // padded LDS row stride of V (see compute_step)
    static constexpr int VBUF = STEP * VSTRIDE;      // per-wave V staging bytes
    static constexpr int HB = 16;                    // query heads per matrix block
    static_assert(NW * HB * (D + 2) * 4 <= NW * VBUF, "merge scratch must fit");
};

// Layout of one cache row in memory: bf16 (2 bytes per element) or fp8 e4m3
// codes (1 byte). Each lane loads K 16 bytes at a time (one MFMA k-step of 8
// elements in bf16, two in fp8) and V 16 bytes per wave-wide load.
template <int D, bool F8>
struct KvFmt {
    static constexpr int RB = F8 ? D : 2 * D;               // bytes per cache row
    static constexpr int KLOADS = RB / 64;                  // K loads per lane per 16-row half
    static constexpr int VCPR = RB / 16;                    // 16-byte chunks per row
    static constexpr int VRPI = 64 / VCPR;                  // rows per wave-wide V load
    static constexpr int VLOADS = MfmaCfg<D>::STEP / VRPI;  // V loads per lane per step
};

// The lane index as a value the compiler must recompute where it is used:
// addresses derived from it in rarely taken code are then not hoisted out of
// the hot loop (where they would hold registers for its whole length).
__device__ __forceinline__ int opaque_lane(int lane) {
    asm volatile("" : "+v"(lane));
    return lane;
}
// x of lane src (0..63)
__device__ __forceinline__ float shfl_from(float x, int src) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, x)));
}

__device__ __forceinline__ int kslot(int qd, int e) { return e < 4 ? 4 * qd + e : 12 + 4 * qd + e; }

// One wave's running state for 16 query heads.
template <int D>
struct MfmaState {
    f32x4_t acc[MfmaCfg<D>::NB];  // O[head 4qd+v][x = 16nb + r], unnormalised
    float m_ref;                  // reference max of head r (log2 units), equal in the 4 qd lanes
    float l_lane;                 // this lane's share of head r's running sum
    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int nb = 0; nb < MfmaCfg<D>::NB; nb++) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m_ref = -INFINITY;
        l_lane = 0.f;
    }
};

// Q^T operand of query head `hq`: for k-step k lane holds Q[hq][d0 .. d0+8],
// d0 = 32k + 8qd, in the order the K operand's lanes hold K's elements. With
// a one-byte cache (fp8 or int8 codes) a lane's 16-byte K load holds 16 elements, which feed two
// k-steps: then d0 = 16qd + 8(k%2) + 64(k/2) (any order of d gives the same
// dot product, as long as Q and K agree).
template <int D, bool F8 = false>
__device__ __forceinline__ void load_q_operand(const uint16_t *__restrict__ q, size_t qrow,
                                               int qd, bf16x8_t (&qop)[MfmaCfg<D>::KSTEPS]) {
#pragma unroll
    for (int k = 0; k < MfmaCfg<D>::KSTEPS; k++) {
        const int d0 = F8 ? 16 * qd + 8 * (k & 1) + 64 * (k >> 1) : 32 * k + 8 * qd;
        qop[k] = *(const bf16x8_t *)(q + qrow * D + d0);
    }
}

// 16 fp8 e4m3 codes (4 dwords, element e in byte e) -> elements 0..7 and
// 8..15 as bf16, two codes per instruction (v_cvt_scalef32_pk_bf16_fp8 with
// scale 1: the low half of the result is byte 0 (word select: byte 2), the
// high half byte 1 (byte 3); exact, since every e4m3 value is a bf16 value —
// measured on the device for all 256 codes against the fp32 conversion).
__device__ __forceinline__ void fp8x16_to_bf16(const u32x4_t &w, bf16x8_t &lo, bf16x8_t &hi) {
    uint32_t o[8];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        // (a scalar copy first: a bit cast of a vector element expression
        // reads element 0 with this compiler)
        const uint32_t wk = w[k];
        o[2 * k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wk, 1.0f, false));
        o[2 * k + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wk, 1.0f, true));
    }
    lo = __builtin_bit_cast(bf16x8_t, (u32x4_t){o[0], o[1], o[2], o[3]});
    hi = __builtin_bit_cast(bf16x8_t, (u32x4_t){o[4], o[5], o[6], o[7]});
}

// 16 int8 codes (two's complement, element e in byte e) -> elements 0..7
// and 8..15 as bf16: each byte sign-extended to fp32 (one conversion with a
// byte select), pairs packed to bf16. Exact: a code's magnitude is at most
// 128, which needs at most 8 significant bits.
__device__ __forceinline__ void int8x16_to_bf16(const u32x4_t &w, bf16x8_t &lo, bf16x8_t &hi) {
    uint32_t o[8];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const uint32_t wk = w[k];  // (a scalar copy, as in fp8x16_to_bf16)
#pragma unroll
        for (int p = 0; p < 2; p++) {
            const float f0 = (float)(int8_t)(wk >> (16 * p)), f1 = (float)(int8_t)(wk >> (16 * p + 8));
            const bf16x2_t v = {(__bf16)f0, (__bf16)f1};
            o[2 * k + p] = __builtin_bit_cast(uint32_t, v);
        }
    }
    lo = __builtin_bit_cast(bf16x8_t, (u32x4_t){o[0], o[1], o[2], o[3]});
    hi = __builtin_bit_cast(bf16x8_t, (u32x4_t){o[4], o[5], o[6], o[7]});
}

// 16 one-byte codes of a cache of fp8 (I8 false) or int8 codes -> bf16.
template <bool I8>
__device__ __forceinline__ void codes16_to_bf16(const u32x4_t &w, bf16x8_t &lo, bf16x8_t &hi) {
    if constexpr (I8)
        int8x16_to_bf16(w, lo, hi);
    else
        fp8x16_to_bf16(w, lo, hi);
}

// K and V of one 32-position step as loaded: K in the lanes of the A operand
// of the score MFMA (bf16: the operand itself), V row-contiguous (16 bytes
// per lane).
template <int D, bool F8 = false>
struct StepData {
    u32x4_t kraw[2][KvFmt<D, F8>::KLOADS];  // per 16-row half
    u32x4_t vld[KvFmt<D, F8>::VLOADS];
};

// Where the K/V rows of one 32-position step come from: for each 16-row half,
// a buffer descriptor and the byte offset of the half's first row in it.
// Rows past a descriptor's extent come back as zeros without a memory access
// (and are masked later), so a step past the end loads nothing.
struct StepSrc {
    rsrc_t k[2], v[2];
    uint32_t off[2];
};

// Contiguous cache [b][g][S][d]: both halves in the head's S rows, the
// descriptors' extent the sequence length.
template <int D, bool F8 = false, bool I8 = false>
struct ContigKV {
    static constexpr bool kPaged = false;
    static constexpr bool kF8 = F8;  // one byte per element (fp8 or int8 codes)
    static constexpr bool kI8 = I8;  // the codes are int8
    static_assert(F8 || !I8, "int8 codes are one byte");
    static constexpr int kStage = 1;
    const uint8_t *k, *v;
    int g, S;
    __device__ __forceinline__ StepSrc step(int i, int j, int L, int t0, bool &) const {
        constexpr uint32_t RB = KvFmt<D, F8>::RB;
        const size_t head = ((size_t)i * g + j) * (size_t)S * RB;
        const rsrc_t kr = make_rsrc(k + head, (uint32_t)L * RB);
        const rsrc_t vr = make_rsrc(v + head, (uint32_t)L * RB);
        return StepSrc{{kr, kr}, {vr, vr}, {(uint32_t)t0 * RB, (uint32_t)(t0 + 16) * RB}};
    }
    __device__ __forceinline__ StepSrc none() const {
        const rsrc_t z = make_rsrc(k, 0);
        return StepSrc{{z, z}, {z, z}, {0u, 0u}};
    }
};

// Paged cache: pages [num_pages][g][P][d], position t of sequence i in row
// t % P of page block_table[i][t / P] ([MQA blog] §3.3). P is a multiple of
// 16, so each half of a step lies in one page. A referenced page id outside
// [0, num_pages) reads nothing and sets `bad`. The kernels stage the page ids
// of their steps in LDS (up to kStage entries, two per step; further steps
// look the table up) before the first step, so that no table lookup sits
// between a claim and its loads.
template <int D, bool F8 = false, bool I8 = false>
struct PagedKV {
    static constexpr bool kPaged = true;
    static constexpr bool kF8 = F8;  // one byte per element (fp8 or int8 codes)
    static constexpr bool kI8 = I8;  // the codes are int8
    static_assert(F8 || !I8, "int8 codes are one byte");
    static constexpr int kStage = F8 ? 1024 : 4096;  // (fp8: eight waves' buffers share the LDS)
    const uint8_t *k, *v;
    const int32_t *bt;
    int g, P, max_pages, num_pages;
    // page id of position `row` of sequence i (-1 at or past L)
    __device__ __forceinline__ int page_id(int i, int row, int L) const {
        return row < L ? bt[(size_t)i * max_pages + row / P] : -1;
    }
    // the step at t0 of K/V head j, its halves in pages id0 and id1
    __device__ __forceinline__ StepSrc step_ids(int j, int L, int t0, int id0, int id1,
                                                bool &bad) const {
        constexpr uint32_t RB = KvFmt<D, F8>::RB;
        StepSrc s;
#pragma unroll
        for (int hf = 0; hf < 2; hf++) {
            const int row = t0 + 16 * hf;
            const int pid = hf ? id1 : id0;
            const bool ok = row < L && pid >= 0 && pid < num_pages;
            bad |= row < L && !ok;
            // the extent stops at the sequence's length, so rows of the page
            // past it (stale or never written) are never read: they load as 0
            const uint32_t rows = ok ? (uint32_t)min(P, L - row / P * P) : 0u;
            const size_t page = ((size_t)(ok ? pid : 0) * g + j) * (size_t)P * RB;
            s.k[hf] = make_rsrc(k + page, rows * RB);
            s.v[hf] = make_rsrc(v + page, rows * RB);
            s.off[hf] = (uint32_t)(row % P) * RB;
        }
        return s;
    }
    __device__ __forceinline__ StepSrc none() const {
        const rsrc_t z = make_rsrc(k, 0);
        return StepSrc{{z, z}, {z, z}, {0u, 0u}};
    }
};

// Stage the page ids of entries 0..n-1 into pg (where(e, i, row, L): entry
// e is position row of sequence i, of length L), whole work-group, four
// lookups in flight per thread; the caller's barrier publishes them.
template <int NT, class KV, class Where>
__device__ __forceinline__ void stage_page_ids(const KV &kv, int *pg, int n, Where where) {
    for (int e0 = threadIdx.x; e0 < n; e0 += 4 * NT) {
        int id[4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const int e = e0 + k * NT;
            id[k] = -1;
            if (e < n) {
                int i, row, L;
                where(e, i, row, L);
                id[k] = kv.page_id(i, row, L);
            }
        }
#pragma unroll
        for (int k = 0; k < 4; k++)
            if (e0 + k * NT < n) pg[e0 + k * NT] = id[k];
    }
}

// Issue the loads of one step: streamed (non-temporal), or with SHARED
// cached, for steps that another group of waves reads again right after.
template <int D, bool F8 = false, bool SHARED = false>
__device__ __forceinline__ void load_step(const StepSrc &src, int lane, StepData<D, F8> &sd) {
    auto ld = [](rsrc_t r, uint32_t off) __attribute__((always_inline)) {
        return SHARED ? buffer_cached16(r, off) : buffer_stream16(r, off);
    };
    using F = KvFmt<D, F8>;
    const int r = lane & 15, qd = lane >> 4;
    const int vl_row = lane / F::VCPR, vl_chunk = lane % F::VCPR;
    const uint32_t kl = r * F::RB + 16 * qd;
    const uint32_t vl = vl_row * F::RB + 16 * vl_chunk;
#pragma unroll
    for (int pb = 0; pb < 2; pb++)
#pragma unroll
        for (int k = 0; k < F::KLOADS; k++)
            sd.kraw[pb][k] = ld(src.k[pb], src.off[pb] + kl + 64 * k);
#pragma unroll
    for (int ii = 0; ii < F::VLOADS; ii++) {
        constexpr int H = 16 / F::VRPI;  // V loads per half
        sd.vld[ii] = ld(src.v[ii / H], src.off[ii / H] + vl + (ii % H) * F::VRPI * F::RB);
    }
}

// A step that read an invalid page: its unit's results become NaN (the state's
// sum is NaN, which every merge carries) and the error flag is raised.
template <int D, int NHB>
__device__ __forceinline__ void poison_state(MfmaState<D> (&st)[NHB], int32_t *err, int lane) {
#pragma unroll
    for (int hb = 0; hb < NHB; hb++) st[hb].l_lane = __builtin_nanf("");
    if (err && lane == 0) atomicOr(err, MQA_DEVERR_PAGE);
}

// V rows of the step at t0 into the wave's staging buffer vb (rows at or
// past t_end zeroed: they may hold anything, NaN included). Done before the
// next step's loads are issued, so that this step's V registers are free for
// them (the wave then holds one step of V in registers, not two).
template <int D, bool F8, bool I8>
__device__ __forceinline__ void stage_v_rows(const StepData<D, F8> &sd, int t0, int t_end,
                                             uint8_t *vb, int lane) {
    using C = MfmaCfg<D>;
    using F = KvFmt<D, F8>;
    const int vl_row = lane / F::VCPR, vl_chunk = lane % F::VCPR;
    const bool tail = t0 + C::STEP > t_end;  // wave-uniform
#pragma unroll
    for (int ii = 0; ii < F::VLOADS; ii++) {
        const int row = ii * F::VRPI + vl_row;
        u32x4_t v = sd.vld[ii];
        if (tail && t0 + row >= t_end) v = u32x4_t{0u, 0u, 0u, 0u};
        if constexpr (F8) {  // 16 codes -> 16 bf16 (32 bytes) of the row
            bf16x8_t lo, hi;
            codes16_to_bf16<I8>(v, lo, hi);
            *(bf16x8_t *)(vb + row * C::VSTRIDE + 32 * vl_chunk) = lo;
            *(bf16x8_t *)(vb + row * C::VSTRIDE + 32 * vl_chunk + 16) = hi;
        } else {
            *(u32x4_t *)(vb + row * C::VSTRIDE + 16 * vl_chunk) = v;
        }
    }
}
template <int D, bool F8, bool I8 = false>
__device__ __forceinline__ void stage_v(const StepData<D, F8> &sd, int t0, int t_end, uint8_t *vb,
                                        int lane) {
    if (t0 + MfmaCfg<D>::STEP > t_end)  // wave-uniform: a real branch
        stage_v_rows<D, F8, I8>(sd, t0, t_end, vb, lane);
    else
        stage_v_rows<D, F8, I8>(sd, t0, 0x7fffffff, vb, lane);
}

// One 32-position step [t0, t0+32) of one wave from loaded data, rows >=
// t_end masked; vb is the wave's staging buffer, which already holds the
// step's V rows (stage_v). The wave computes NHB blocks
// of 16 query rows against the same K and V registers (block b: its q
// operand qop[b] and state st[b]), so the K/V bytes are loaded once for all
// of them. MULTI (several query tokens per sequence): query row r of block b
// also stops at its own t_row[b] (its token's causal end, per lane, <=
// t_end); t_lo is the smallest t_row of the wave. A row can then have no
// position in a step, so exponentials of masked scores are set to 0 (not
// exp2(-inf - -inf)). With a sliding window row r also starts at t_rs[hb]
// (per lane); t_hs is the latest start of the wave (0: no window).
// MASKED: the step may hold masked positions (a tail past the earliest end,
// or a head before the latest start); the other steps skip every mask test.
template <int D, bool MULTI, int NHB, bool F8, bool MASKED, bool I8>
__device__ __forceinline__ void compute_step_v(const StepData<D, F8> &sd, int t0, int t_end, int t_lo,
                                               const int (&t_row)[NHB], int t_hs,
                                               const int (&t_rs)[NHB],
                                               const bf16x8_t (&qop)[NHB][MfmaCfg<D>::KSTEPS],
                                               MfmaState<D> (&st)[NHB], uint8_t *vb, int lane,
                                               float qk_scale_log2) {
    using C = MfmaCfg<D>;
    using F = KvFmt<D, F8>;
    const int r = lane & 15, qd = lane >> 4;
    const bool tail = MASKED && t0 + C::STEP > (MULTI ? t_lo : t_end);
    const bool head = MASKED && MULTI && t0 < t_hs;  // wave-uniform
    // K operands (fp8: decoded to bf16 here; the scales are applied outside)
    bf16x8_t kop[2][C::KSTEPS];
#pragma unroll
    for (int pb = 0; pb < 2; pb++)
#pragma unroll
        for (int k = 0; k < F::KLOADS; k++) {
            if constexpr (F8)
                codes16_to_bf16<I8>(sd.kraw[pb][k], kop[pb][2 * k], kop[pb][2 * k + 1]);
            else
                kop[pb][k] = __builtin_bit_cast(bf16x8_t, sd.kraw[pb][k]);
        }

    // ---- scores ----
    float s2[NHB][8];
#pragma unroll
    for (int hb = 0; hb < NHB; hb++) {
        f32x4_t sc[2];
#pragma unroll
        for (int pb = 0; pb < 2; pb++) {
            sc[pb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < C::KSTEPS; k++)
                sc[pb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[pb][k], qop[hb][k], sc[pb], 0,
                                                                 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 8; e++) {
            s2[hb][e] = sc[e >> 2][e & 3] * qk_scale_log2;
            const int pos = t0 + kslot(qd, e);
            if ((tail && pos >= (MULTI ? t_row[hb] : t_end)) || (head && pos < t_rs[hb]))
                s2[hb][e] = -INFINITY;
        }
    }

    // ---- online softmax for head r of each block ----
    bf16x8_t phi[NHB], plo[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; hb++) {
        MfmaState<D> &sb = st[hb];
        float smax = s2[hb][0];
#pragma unroll
        for (int e = 1; e < 8; e++) smax = fmaxf(smax, s2[hb][e]);
        if (__any(smax > sb.m_ref + kSlack)) {  // wave-uniform
            // (shuffle addresses built here, not kept live across the whole loop)
            const int ln = opaque_lane(lane);
            float mt = fmaxf(smax, shfl_from(smax, ln ^ 16));
            mt = fmaxf(mt, shfl_from(mt, ln ^ 32));   // max over the head's 32 positions
            mt = fmaxf(mt, sb.m_ref);
            // per head r (several tokens: a row that has seen no position yet
            // keeps its empty state; exp2(-inf - -inf) would be NaN)
            const float alpha = (MULTI && mt == -INFINITY) ? 1.f : fast_exp2(sb.m_ref - mt);
            sb.m_ref = mt;
            sb.l_lane *= alpha;
            // acc rows are heads 4qd+v: fetch their factors from lanes 4qd+v
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const float av = shfl_from(alpha, 4 * (ln >> 4) + v);
#pragma unroll
                for (int nb = 0; nb < C::NB; nb++) sb.acc[nb][v] *= av;
            }
        }
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; e++) {
            p[e] = fast_exp2(s2[hb][e] - sb.m_ref);
            if constexpr (MULTI) p[e] = s2[hb][e] == -INFINITY ? 0.f : p[e];
            sb.l_lane += p[e];
        }
        // P as bf16 hi + lo parts, A operand of the P.V MFMA
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const __bf16 hi = (__bf16)p[e];
            phi[hb][e] = hi;
            plo[hb][e] = (__bf16)(p[e] - (float)hi);
        }
    }

    // ---- P.V (one V operand for every block) ----
    // The B operand wants lane (r, qd) to hold V[kslot(qd, e)][16nb + r],
    // e = 0..7: eight positions of one column, where the staging buffer holds
    // rows. The LDS transpose read gives each lane of a 16-lane group the
    // transpose of what the group loads: lane j gets element j%4 of the
    // 8-byte chunk of group lane 4i + j/4, for i = 0..3 (measured on the
    // device). So lane r of group qd loads row p0 + r/4, columns 16nb +
    // 4(r%4) .. +3, and receives column 16nb + r of rows p0 .. p0+3; two such
    // reads (p0 = 4qd and 16 + 4qd) cover the eight positions. The row stride
    // (ROW_BYTES + 32) puts the four rows of a read in distinct banks.
    const uint8_t *vt = vb + (4 * qd + (r >> 2)) * C::VSTRIDE + 8 * (r & 3);
#pragma unroll
    for (int nb = 0; nb < C::NB; nb++) {
        const i16x4_t v_lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(const lds_u8 *)(vt + 32 * nb));
        const i16x4_t v_hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(const lds_u8 *)(vt + 16 * C::VSTRIDE + 32 * nb));
        const bf16x8_t vop = __builtin_bit_cast(
            bf16x8_t, (i16x8_t){v_lo[0], v_lo[1], v_lo[2], v_lo[3], v_hi[0], v_hi[1], v_hi[2], v_hi[3]});
#pragma unroll
        for (int hb = 0; hb < NHB; hb++) {
            st[hb].acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi[hb], vop, st[hb].acc[nb], 0, 0, 0);
            st[hb].acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo[hb], vop, st[hb].acc[nb], 0, 0, 0);
        }
    }
}

template <int D, bool MULTI, int NHB, bool F8 = false, bool I8 = false>
__device__ __forceinline__ void compute_step(const StepData<D, F8> &sd, int t0, int t_end, int t_lo,
                                             const int (&t_row)[NHB], int t_hs,
                                             const int (&t_rs)[NHB],
                                             const bf16x8_t (&qop)[NHB][MfmaCfg<D>::KSTEPS],
                                             MfmaState<D> (&st)[NHB], uint8_t *vb, int lane,
                                             float qk_scale_log2) {
    // wave-uniform: a real branch between the two forms
    const bool masked = t0 + MfmaCfg<D>::STEP > (MULTI ? t_lo : t_end) || (MULTI && t0 < t_hs);
    if (masked)
        compute_step_v<D, MULTI, NHB, F8, true, I8>(sd, t0, t_end, t_lo, t_row, t_hs, t_rs, qop, st,
                                                    vb, lane, qk_scale_log2);
    else
        compute_step_v<D, MULTI, NHB, F8, false, I8>(sd, t0, t_end, t_lo, t_row, t_hs, t_rs, qop, st,
                                                     vb, lane, qk_scale_log2);
}

// Query rows of a unit (sequence i, K/V head j). With T query tokens per
// sequence (MULTI) a unit has R = T * Gh rows, row rho = tau * Gh + head,
// q and out are [b][T][h][d], and token tau (position L - T + tau) sees the
// positions t <= L - T + tau: the causal mask stays per query position when
// K/V heads are shared ([GQA notes] §十 item 10). Otherwise R = Gh and every
// row sees t < L.
// A sliding window of W positions (W > 0; only with MULTI) keeps, for the
// query at position p, the positions t in (p - W, p]: the window start
// replaces 0 ([MQA concept] 玩家對比: GQA with a sliding window). The first
// 32-position step any row of a length-L sequence sees:
__device__ __forceinline__ int window_first_step(int L, int T, int W) {
    return W > 0 ? max(0, L - T + 1 - W) / 32 : 0;
}

template <bool MULTI>
struct QRows {
    int T, Gh, h;
    int W;  // sliding window (0: none)
    __device__ __forceinline__ int tok(int rho) const { return MULTI ? rho / Gh : 0; }
    __device__ __forceinline__ int first_step(int L) const {
        if constexpr (MULTI)
            return window_first_step(L, T, W);
        else
            return 0;
    }
    // first position row rho of a length-L sequence sees
    __device__ __forceinline__ int row_start(int L, int rho) const {
        if constexpr (MULTI)
            return W > 0 ? max(0, L - T + 1 + rho / Gh - W) : 0;
        else
            return 0;
    }
    __device__ __forceinline__ size_t row(int i, int j, int rho) const {
        if constexpr (MULTI)
            return ((size_t)i * T + rho / Gh) * h + (size_t)j * Gh + rho % Gh;
        else
            return (size_t)i * h + (size_t)j * Gh + rho;
    }
};

// Steps s_begin, s_begin+stride, ... < s_end (src(step, bad) gives where a
// step's rows are), with the loads of the next NBUF-1 steps in flight while
// one computes (NBUF register sets in rotation; the loop is unrolled by NBUF
// so that each set keeps fixed registers). Past the last step a prefetch
// asks for nothing.
template <int D, bool MULTI, int NHB, int NBUF, bool F8, bool I8, class Src>
__device__ __forceinline__ void run_steps(const Src &src, const StepSrc &nothing, int s_begin,
                                          int s_end, int stride, int t_end, int t_lo,
                                          const int (&t_row)[NHB], int t_hs,
                                          const int (&t_rs)[NHB],
                                          const bf16x8_t (&qop)[NHB][MfmaCfg<D>::KSTEPS],
                                          MfmaState<D> (&st)[NHB], uint8_t *vb, int lane,
                                          float qk_scale_log2, int32_t *err) {
    using C = MfmaCfg<D>;
    static_assert(NBUF >= 2, "at least one step in flight");
    int stp = s_begin;
    if (stp >= s_end) return;
    StepData<D, F8> buf[NBUF];
    bool bad[NBUF];
#pragma unroll
    for (int k = 0; k < NBUF - 1; k++) {
        const int sk = stp + k * stride;
        bad[k] = false;
        load_step<D, F8>(sk < s_end ? src(sk, bad[k]) : nothing, lane, buf[k]);
    }
    while (true) {
#pragma unroll
        for (int k = 0; k < NBUF; k++) {
            // the step NBUF-1 ahead, into the set computed last
            const int kn = (k + NBUF - 1) % NBUF;
            const int sn = stp + (NBUF - 1) * stride;
            stage_v<D, F8, I8>(buf[k], stp * C::STEP, t_end, vb, lane);
            bad[kn] = false;
            load_step<D, F8>(sn < s_end ? src(sn, bad[kn]) : nothing, lane, buf[kn]);
            compute_step<D, MULTI, NHB, F8, I8>(buf[k], stp * C::STEP, t_end, t_lo, t_row, t_hs,
                                                t_rs, qop, st, vb, lane, qk_scale_log2);
            if (bad[k]) poison_state<D>(st, err, lane);
            stp += stride;
            if (stp >= s_end) return;
        }
    }
}

// Merge of the running states of the waves that share one 16-row block of a
// partition, in two halves around a work-group barrier. First every wave
// stores its state in lane order: acc in so[slot][nb][lane] (16 bytes per lane
// and column block) and (reference max, sum) of head r in sml[slot][r].
template <int D>
__device__ __forceinline__ void publish_lanes(const MfmaState<D> &st, f32x4_t *so, float2 *sml, int slot,
                                              int lane) {
    using C = MfmaCfg<D>;
    const int r = lane & 15, qd = lane >> 4;
    const float l_head = st.l_lane + __shfl_xor(st.l_lane, 16);
    const float l_tot = l_head + __shfl_xor(l_head, 32);
#pragma unroll
    for (int nb = 0; nb < C::NB; nb++) so[(slot * C::NB + nb) * 64 + lane] = st.acc[nb];
    if (qd == 0) sml[slot * C::HB + r] = make_float2(st.m_ref, l_tot);
}

// Then wave `part` of the block's `nparts` merges column blocks nb = part,
// part + nparts, ... of the NSRC published states: lane (r, qd) holds rows
// 4qd .. 4qd+3 of the block in column 16nb + r of every source, rescaled to
// the largest reference max (a source that saw no position, max -inf, weighs
// 0). Row rho0 + 4qd + v (< R; rows past R pad the block and are dropped) of
// the partition goes to part_o[((row0 + rho) * nsplit + s) * D + col] times
// vsc, its (max, sum) to part_ml[(row0 + rho) * nsplit + s] (part 0), where
// row0 is the unit's first partial row: the layout combine_kernel reads.
template <int D, int NSRC>
__device__ __forceinline__ void merge_lanes(const f32x4_t *so, const float2 *sml, int part, int nparts,
                                            int lane, float vsc, int rho0, int R, size_t row0, int nsplit,
                                            int s, float *__restrict__ part_o,
                                            float2 *__restrict__ part_ml) {
    using C = MfmaCfg<D>;
    const int r = lane & 15, qd = lane >> 4;
    float Ms[NSRC][4], Ls[NSRC][4], Mx[4];
#pragma unroll
    for (int v = 0; v < 4; v++) Mx[v] = -INFINITY;
#pragma unroll
    for (int src = 0; src < NSRC; src++) {
        const f32x4_t a = *(const f32x4_t *)&sml[src * C::HB + 4 * qd];
        const f32x4_t c = *(const f32x4_t *)&sml[src * C::HB + 4 * qd + 2];
        Ms[src][0] = a[0], Ls[src][0] = a[1], Ms[src][1] = a[2], Ls[src][1] = a[3];
        Ms[src][2] = c[0], Ls[src][2] = c[1], Ms[src][3] = c[2], Ls[src][3] = c[3];
#pragma unroll
        for (int v = 0; v < 4; v++) Mx[v] = fmaxf(Mx[v], Ms[src][v]);
    }
    float wt[NSRC][4], Lt[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int src = 0; src < NSRC; src++)
#pragma unroll
        for (int v = 0; v < 4; v++) {
            wt[src][v] = Ms[src][v] == -INFINITY ? 0.f : fast_exp2(Ms[src][v] - Mx[v]);
            Lt[v] = fmaf(wt[src][v], Ls[src][v], Lt[v]);
        }
    for (int nb = part; nb < C::NB; nb += nparts) {
        f32x4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int src = 0; src < NSRC; src++) {
            const f32x4_t a = so[(src * C::NB + nb) * 64 + lane];
#pragma unroll
            for (int v = 0; v < 4; v++) o[v] = fmaf(wt[src][v], a[v], o[v]);
        }
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const int rho = rho0 + 4 * qd + v;
            if (rho < R) part_o[((row0 + rho) * nsplit + s) * D + 16 * nb + r] = o[v] * vsc;
        }
    }
    if (part == 0 && r == 0) {
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const int rho = rho0 + 4 * qd + v;
            if (rho < R) part_ml[(row0 + rho) * nsplit + s] = make_float2(Mx[v], Lt[v]);
        }
    }
}

// Fixed partitions: one work-group per (partition of split_chunk positions,
// K/V head, group of NHB blocks of 16 query rows, sequence); writes partials
// for the log-sum-exp combine (partial row (i*g + j)*R + rho).
template <int D, class KV, bool MULTI, int NHB>
__global__ void __launch_bounds__(256)
split_mfma_kernel(const uint16_t *__restrict__ q, const KV kv, const int32_t *__restrict__ seq_lens,
                  const QRows<MULTI> qr, int g, int S, int R, int ngroups, int chunk, int nsplit,
                  float qk_base, const float *__restrict__ k_scale,
                  const float *__restrict__ v_scale, float *__restrict__ part_o,
                  float2 *__restrict__ part_ml, int32_t *__restrict__ err) {
    using C = MfmaCfg<D>;
    constexpr bool F8 = KV::kF8;
    __shared__ __attribute__((aligned(16))) uint8_t vbuf[C::NW][C::VBUF];
    __shared__ int pg[KV::kStage];  // paged: the page ids of the partition's steps

    const int s = blockIdx.x;
    const int j = blockIdx.y / ngroups;
    const int hg = blockIdx.y % ngroups;  // blocks hg*NHB .. hg*NHB+NHB-1
    const int i = blockIdx.z;
    const int L = seq_lens[i];
    if (L < qr.T || L > S) return;  // reported by the combine
    // partitions are counted from the first step any row sees (position 0
    // without a window), so a window leaves none of them empty
    const int t_begin = qr.first_step(L) * C::STEP + s * chunk;
    if (t_begin >= L) return;
    const int t_end = min(t_begin + chunk, L);
    const int s0 = t_begin / C::STEP;  // steps numbered from the sequence start
    const int nsteps = (t_end + C::STEP - 1) / C::STEP - s0;

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, qd = lane >> 4;

    // padded rows reuse the last real one and are never written out
    bf16x8_t qop[NHB][C::KSTEPS];
    int t_row[NHB], t_rs[NHB];  // causal ends and window starts: this lane's row in each block
#pragma unroll
    for (int b = 0; b < NHB; b++) {
        const int rho = min((hg * NHB + b) * C::HB + r, R - 1);
        load_q_operand<D, F8>(q, qr.row(i, j, rho), qd, qop[b]);
        t_row[b] = min(t_end, L - qr.T + 1 + qr.tok(rho));
        t_rs[b] = qr.row_start(L, rho);
    }
    const int t_lo = min(t_end, L - qr.T + 1);  // the earliest end of the wave
    const int t_hs = qr.row_start(L, R - 1);     // and the latest start

    const int ne = KV::kPaged ? min(2 * nsteps, KV::kStage) : 0;
    if constexpr (KV::kPaged) {
        stage_page_ids<256>(kv, pg, ne, [&](int e, int &i_, int &row, int &L_) {
            i_ = i;
            row = s0 * C::STEP + 16 * e;
            L_ = L;
        });
        __syncthreads();
    }
    auto src = [&](int stp, bool &bad) __attribute__((always_inline)) {
        const int t0 = stp * C::STEP;
        if constexpr (KV::kPaged) {
            const int e = 2 * (stp - s0);
            int id0, id1;
            if (e < ne) {
                id0 = pg[e];
                id1 = pg[e + 1];
            } else {  // past what LDS holds: look the ids up
                id0 = kv.page_id(i, t0, L);
                id1 = kv.page_id(i, t0 + 16, L);
            }
            return kv.step_ids(j, L, t0, __builtin_amdgcn_readfirstlane(id0),
                               __builtin_amdgcn_readfirstlane(id1), bad);
        } else {
            return kv.step(i, j, L, t0, bad);
        }
    };

    MfmaState<D> st[NHB];
#pragma unroll
    for (int b = 0; b < NHB; b++) st[b].reset();
    // a code cache (fp8, int8): scores scale by the head's K scale, outputs by its V scale
    const float qk_scale_log2 = F8 ? qk_base * k_scale[j] : qk_base;
    const float vsc = F8 ? v_scale[j] : 1.f;
    run_steps<D, MULTI, NHB, 2, F8, KV::kI8>(src, kv.none(), s0 + w, s0 + nsteps, C::NW, t_end,
                                             t_lo, t_row, t_hs, t_rs, qop, st, vbuf[w], lane,
                                             qk_scale_log2, err);

    // merge the waves' states block by block through the staging buffers;
    // wave w writes column blocks w, w + NW, ...
    f32x4_t *so = (f32x4_t *)&vbuf[0][0];
    float2 *sml = (float2 *)(so + C::NW * C::NB * 64);
    static_assert(C::NW * C::NB * 64 * 16 + C::NW * C::HB * 8 <= C::NW * C::VBUF, "merge scratch must fit");
    const size_t row0 = ((size_t)i * g + j) * R;  // the unit's first partial row
#pragma unroll
    for (int b = 0; b < NHB; b++) {
        const int hb = hg * NHB + b;
        __syncthreads();  // every wave is done with the buffers
        publish_lanes<D>(st[b], so, sml, w, lane);
        __syncthreads();
        merge_lanes<D, C::NW>(so, sml, w, C::NW, lane, vsc, hb * C::HB, R, row0, nsplit, s, part_o, part_ml);
    }
}

// Fixed partitions for units of more than 16 query rows: one work-group of
// eight waves per (partition, K/V head, pair of 16-row blocks, sequence).
// Waves w and w+4 form a pair that takes the partition's steps w%4, w%4 + 4,
// ... for blocks 2hg and 2hg+1. The pair's loader (w < 4) loads each step
// once and writes its K (in the score MFMA's operand order, 16 bytes per
// lane) and its V rows (the staging layout of the transpose reads) into one
// of the pair's two LDS buffers; after a work-group barrier both waves read
// the step from there and compute their own block. Each wave then needs one
// block's registers, so every SIMD holds two waves (a loader and a reader)
// whose latencies overlap, and the K/V bytes still leave HBM once.
template <int D, class KV, bool MULTI>
__global__ void __launch_bounds__(512)
split_pair_kernel(const uint16_t *__restrict__ q, const KV kv, const int32_t *__restrict__ seq_lens,
                  const QRows<MULTI> qr, int g, int S, int R, int ngroups, int chunk, int nsplit,
                  float qk_base, const float *__restrict__ k_scale,
                  const float *__restrict__ v_scale, float *__restrict__ part_o,
                  float2 *__restrict__ part_ml, int32_t *__restrict__ err) {
    using C = MfmaCfg<D>;
    using F = KvFmt<D, KV::kF8>;
    constexpr bool F8 = KV::kF8;
    constexpr int KBYTES = 2 * F::KLOADS * 64 * 16;  // one step's K, operand order
    constexpr int BUF = KBYTES + C::VBUF + 16;        // + V rows + the step's bad-page flag
    static_assert(8 * C::HB * (D + 2) * 4 <= 4 * 2 * BUF, "merge scratch must fit");
    __shared__ __attribute__((aligned(16))) uint8_t lds[4][2][BUF];
    __shared__ int pg[KV::kStage];  // paged: the page ids of the partition's steps

    const int s = blockIdx.x;
    const int j = blockIdx.y / ngroups;
    const int hg = blockIdx.y % ngroups;  // blocks 2hg, 2hg+1
    const int i = blockIdx.z;
    const int L = seq_lens[i];
    if (L < qr.T || L > S) return;  // reported by the combine
    const int t_begin = qr.first_step(L) * C::STEP + s * chunk;
    if (t_begin >= L) return;
    const int t_end = min(t_begin + chunk, L);
    const int s0 = t_begin / C::STEP;
    const int nsteps = (t_end + C::STEP - 1) / C::STEP - s0;

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, qd = lane >> 4;
    const int pair = w % 4;
    const bool loader = w < 4;
    const int hb = hg * 2 + w / 4;  // this wave's block
    const bool rows = hb * C::HB < R;

    bf16x8_t qop[1][C::KSTEPS];
    int t_row[1], t_rs[1];
    {
        const int rho = min(hb * C::HB + r, R - 1);  // padded rows reuse the last real one
        load_q_operand<D, F8>(q, qr.row(i, j, rho), qd, qop[0]);
        t_row[0] = min(t_end, L - qr.T + 1 + qr.tok(rho));
        t_rs[0] = qr.row_start(L, rho);
    }
    const int t_lo = min(t_end, L - qr.T + 1);
    const int t_hs = qr.row_start(L, R - 1);

    const int ne = KV::kPaged ? min(2 * nsteps, KV::kStage) : 0;
    if constexpr (KV::kPaged) {
        stage_page_ids<512>(kv, pg, ne, [&](int e, int &i_, int &row, int &L_) {
            i_ = i;
            row = s0 * C::STEP + 16 * e;
            L_ = L;
        });
        __syncthreads();
    }
    auto src = [&](int stp, bool &bad) __attribute__((always_inline)) {
        const int t0 = stp * C::STEP;
        if constexpr (KV::kPaged) {
            const int e = 2 * (stp - s0);
            int id0, id1;
            if (e < ne) {
                id0 = pg[e];
                id1 = pg[e + 1];
            } else {
                id0 = kv.page_id(i, t0, L);
                id1 = kv.page_id(i, t0 + 16, L);
            }
            return kv.step_ids(j, L, t0, __builtin_amdgcn_readfirstlane(id0),
                               __builtin_amdgcn_readfirstlane(id1), bad);
        } else {
            return kv.step(i, j, L, t0, bad);
        }
    };

    MfmaState<D> st[1];
    st[0].reset();
    const float qk_scale_log2 = F8 ? qk_base * k_scale[j] : qk_base;
    const float vsc = F8 ? v_scale[j] : 1.f;
    // every wave runs the same number of iterations (one barrier each)
    const int niter = (nsteps + 3) / 4;
    StepData<D, F8> nxt;  // the loader's step in flight
    bool bad_nxt = false;
    if (loader) load_step<D, F8>(pair < nsteps ? src(s0 + pair, bad_nxt) : kv.none(), lane, nxt);
    for (int it = 0; it < niter; it++) {
        const int stp = s0 + pair + 4 * it;
        const bool have = stp < s0 + nsteps;  // wave-uniform
        uint8_t *buf = lds[pair][it & 1];
        if (loader) {
            if (have) {
#pragma unroll
                for (int pb = 0; pb < 2; pb++)
#pragma unroll
                    for (int k = 0; k < F::KLOADS; k++)
                        *(u32x4_t *)(buf + ((pb * F::KLOADS + k) * 64 + lane) * 16) = nxt.kraw[pb][k];
                stage_v<D, F8, KV::kI8>(nxt, stp * C::STEP, t_end, buf + KBYTES, lane);
                if (lane == 0) *(int *)(buf + KBYTES + C::VBUF) = bad_nxt ? 1 : 0;
            }
            const int sn = stp + 4;
            bad_nxt = false;
            load_step<D, F8>(sn < s0 + nsteps ? src(sn, bad_nxt) : kv.none(), lane, nxt);
        }
        __syncthreads();  // the pair's buffer holds step stp
        if (have && rows) {
            StepData<D, F8> cur;
#pragma unroll
            for (int pb = 0; pb < 2; pb++)
#pragma unroll
                for (int k = 0; k < F::KLOADS; k++)
                    cur.kraw[pb][k] = *(const u32x4_t *)(buf + ((pb * F::KLOADS + k) * 64 + lane) * 16);
            compute_step<D, MULTI, 1, F8, KV::kI8>(cur, stp * C::STEP, t_end, t_lo, t_row, t_hs,
                                                   t_rs, qop, st, buf + KBYTES, lane,
                                                   qk_scale_log2);
            if (*(const int *)(buf + KBYTES + C::VBUF)) poison_state<D>(st, err, lane);
        }
    }

    // merge the four waves of each block through LDS (slots 0..3: block 2hg,
    // slots 4..7: block 2hg+1); wave w writes column blocks w % 4, w % 4 + 4, ...
    // of its block
    f32x4_t *so = (f32x4_t *)&lds[0][0][0];
    float2 *sml = (float2 *)(so + 8 * C::NB * 64);
    static_assert(8 * C::NB * 64 * 16 + 8 * C::HB * 8 <= 4 * 2 * BUF, "merge scratch must fit");
    __syncthreads();  // every wave is done with the buffers
    publish_lanes<D>(st[0], so, sml, w, lane);
    __syncthreads();
    if (!rows) return;  // a padding block past the unit's rows
    merge_lanes<D, 4>(so + (w / 4) * 4 * C::NB * 64, sml + (w / 4) * 4 * C::HB, w % 4, 4, lane, vsc,
                      hb * C::HB, R, ((size_t)i * g + j) * R, nsplit, s, part_o, part_ml);
}

// ---------------------------------------------------------------------------
// balanced ("stream-K") schedule for the bf16 kernel
// ---------------------------------------------------------------------------
//
// Work unit u = (sequence i, K/V head j) with n_i = ceil(L_i / 32) steps;
// units are numbered i-major and their steps laid end to end (T steps in
// all; sequences with an invalid length contribute none). Work-group w of
// nwg (one per compute unit) takes an equal share of the work whatever the
// lengths (StepSplit: the steps, plus an allowance of C steps per unit for
// closing its segment where a kernel's segment closes are dear; nwg is cut
// on the device so that every range holds >= kStreamMinSteps steps). Its
// waves are split into blocks of 16 query
// heads; with nhb blocks, each block's waves walk the whole range, so the
// blocks read each K/V step at about the same time (the second read comes
// from L2). A unit entirely inside one range is normalised and written to
// `out` directly. A unit cut by range boundaries leaves, for each work-group
// and head block that touch it, a partial (m, l, o) in slot 0 (the range's
// first segment) or slot 1 (its last) and a description of the cut
// (cut_desc); streamk_combine_kernel, launched next, merges the pieces and
// writes `out`.

constexpr int kStreamMaxSeq = 1024;    // sequences per call on this schedule (prefix sums in LDS)
constexpr int kStreamMaxWG = 1024;     // work-groups (bounds the workspace)
constexpr int kStreamMinUnits = 256;   // fewer (sequence, K/V head) units: fixed partitions
constexpr int kStreamMinSteps = 16;    // steps per work-group range, at least
constexpr int kStreamWaves = 4;        // waves per work-group (one work-group per compute unit)
constexpr int kRing = 16;              // segment records per head block

// steps of sequence i (0 for an invalid length: below the T tokens of the
// step, or past the capacity)
__device__ __forceinline__ int seq_steps(int L, int S, int T, int W) {
    return (L < T || L > S) ? 0 : (L + 31) / 32 - window_first_step(L, T, W);
}

// Exclusive prefixes over sequences, whole work-group (NT threads): steps
// of units, pre[0..b] (units_per_seq units per valid sequence), and valid
// sequences, vpre[0..b]. Each thread takes a contiguous run of sequences;
// the runs are scanned with wave shuffles and the wave totals added. The
// host keeps the step total below 2^31.
template <int NT>
__device__ __forceinline__ void unit_prefix(const int32_t *__restrict__ seq_lens, int b, int S,
                                            int T, int W, int units_per_seq, int *pre, int *vpre,
                                            int *lens, int2 *wtot) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int per = (b + NT - 1) / NT;
    const int a0 = min(b, t * per), a1 = min(b, a0 + per);
    int run = 0, vrun = 0;
    for (int a = a0; a < a1; a++) {
        const int L = seq_lens[a];
        lens[a] = L;  // kept in LDS for the rest of the kernel
        const int n = seq_steps(L, S, T, W);
        run += n;
        vrun += n > 0;
    }
    int v = run, vv = vrun;  // inclusive scans over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(v, off), yy = __shfl_up(vv, off);
        if (lane >= off) {
            v += y;
            vv += yy;
        }
    }
    if (lane == 63) wtot[w] = make_int2(v, vv);
    __syncthreads();
    int acc = v - run, vacc = vv - vrun;
    for (int k = 0; k < w; k++) {
        acc += wtot[k].x;
        vacc += wtot[k].y;
    }
    acc *= units_per_seq;
    for (int a = a0; a < a1; a++) {
        const int n = seq_steps(lens[a], S, T, W);
        pre[a] = acc;
        vpre[a] = vacc;
        acc += n * units_per_seq;
        vacc += n > 0;
    }
    if (t == NT - 1) {
        pre[b] = acc;
        vpre[b] = vacc;
    }
    __syncthreads();
}

// The ranges of the work-groups. Unit (i, j) weighs its n_i steps plus C:
// laid end to end, unit (i, j) takes the weights [U, U + C + n_i) with
// U = pre[i] + C g vpre[i] + j (n_i + C), its allowance first, then its
// steps (step o of the unit at U + C + o); the total is TW = T + C g (valid
// sequences). Work-group w takes the weights [TW w / nwg, TW (w + 1) / nwg)
// and with them every step whose weight falls inside (a boundary inside an
// allowance falls at the unit's first step). A range of at least
// kStreamMinSteps > C weights holds at least one step. With C = 0 this is the
// plain equal split of the steps.
template <int C>
struct StepSplit {
    int T, nwg, g, S, Tq, W, b;
    const int *pre, *vpre, *lens;  // the prefix sums and lengths in LDS
    __device__ __forceinline__ long long useq(int i) const {  // weight before sequence i
        return pre[i] + (long long)C * g * vpre[i];
    }
    // the weight where work-group w's range begins (the total for w = nwg)
    __device__ __forceinline__ long long wstart(int w) const { return useq(b) * w / nwg; }
    // the first step at or after weight wb, for the sequence i that holds it
    // (useq(i) <= wb < useq(i + 1): a sequence with steps)
    __device__ __forceinline__ int step_in(int i, long long wb) const {
        const int n = seq_steps(lens[i], S, Tq, W);
        const long long off = wb - useq(i);
        const int j = (int)(off / (n + C)), o = (int)(off % (n + C));
        return pre[i] + j * n + max(0, o - C);
    }
    // the work-group whose range holds step o of unit (i, j), n steps each
    __device__ __forceinline__ int owner(int i, int j, int n, int o) const {
        const long long TW = useq(b);
        const long long x = useq(i) + (long long)j * (n + C) + C + o;
        return (int)(((x + 1) * nwg - 1) / TW);
    }
};

// Flags between the waves of one work-group, in LDS. A flag is written after
// the data it guards has left the wave (lgkmcnt drained), and the data is read
// only after the flag has been seen; the asm statements also keep the
// compiler from moving LDS accesses across them.
__device__ __forceinline__ void lds_drain() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void lds_flag_set(int *f, int v) {
    __hip_atomic_store(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Wait until *f == v, at most kSpinCap polls (~2^22 * 64 cycles, tens of ms:
// the waits of the claim protocol last at most a few steps of another wave).
// A wait that runs out marks the work-group broken (*broken = 1, stored before
// anything this wave writes to LDS afterwards) and ORs MQA_DEVERR_STALL into
// *err; the caller then goes on, and every row the work-group writes from
// then on is NaN, so that a protocol failure can neither hang the GPU nor
// pass unnoticed. (The loops test a wave-uniform copy of the flag, so that
// they exit uniformly.)
constexpr int kSpinCap = 1 << 22;
__device__ __forceinline__ void lds_flag_wait(int *f, int v, int *broken, int32_t *err) {
    int n = 0;
    while (__builtin_amdgcn_readfirstlane(
               __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) != v) {
        if (++n == kSpinCap) {
            lds_flag_set(broken, 1);
            lds_drain();
            if (err && (threadIdx.x & 63) == 0) atomicOr(err, MQA_DEVERR_STALL);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
}

// One work-group per compute unit, NW waves (four: with 2 steps in flight per
// wave that is ~32 MB in flight on the chip, several times what the memory
// needs to stay busy; more waves only lengthen the queues, measured slower).
// The waves of a head
// block claim the steps of the range one at a time from a counter in LDS, so
// a wave that the hardware serves faster simply takes more steps; the loads
// of a wave's next claimed step are issued before its current step is
// computed, across unit boundaries too. A wave keeps one running state while
// its claims stay in one unit. When its next claim leaves the unit it stores
// the state in its LDS slot and adds (steps done, its bit) to the segment's
// record; the wave whose addition completes the segment's step count merges
// the slots named in the record into its own state and writes the result
// (out, or a partial of a cut unit). No wave waits for another's progress:
// the only waits are for a slot or a record to be released by a merge, and
// each is on a segment that ends earlier in the range, so they cannot form a
// cycle. Which wave computes which step depends on timing, so the rounding
// of the sums can differ between calls.
template <int D, int NW, class KV, bool MULTI, int NHB, bool SHARED = false>
__global__ void __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(1, 8)))
streamk_mfma_kernel(const uint16_t *__restrict__ q, const KV kv,
                    const int32_t *__restrict__ seq_lens, int b, const QRows<MULTI> qr,
                    int g, int S, int R, int ngroups, float qk_base,
                    const float *__restrict__ k_scale, const float *__restrict__ v_scale,
                    float *__restrict__ out, float *__restrict__ part_o,
                    float2 *__restrict__ part_ml, int4 *__restrict__ cut_desc,
                    int32_t *__restrict__ err, int det) {
    using C = MfmaCfg<D>;
    constexpr bool F8 = KV::kF8;  // fp8 or int8 codes: per-K/V-head scales on scores and outputs
    static_assert(NW == 4 || NW == 8, "waves per work-group (the segment records hold 8 bits)");
    __shared__ __attribute__((aligned(16))) uint8_t vbuf[NW][C::VBUF];
    __shared__ f32x4_t slot_o[NW][NHB][C::NB][64];  // a wave's acc, lane-native order
    __shared__ float2 slot_ml[NW][NHB][C::HB];      // (m, l) per head
    __shared__ int slot_busy[NW];              // 1 while the slot holds a state not merged yet
    __shared__ int rec_tag[4][kRing];          // ordinal of the segment the record serves now
    __shared__ uint32_t rec_val[4][kRing];     // (steps done << 8) | waves (bit per wave of the block)
    __shared__ int cursor[4];                  // steps of the range claimed so far, per head group
    __shared__ int first_seq, last_seq;        // sequences holding the range's first and last steps
    __shared__ int range_end[2];               // the range's first step and the next range's
    __shared__ int broken;                     // 1 once a wait between waves ran out (lds_flag_wait)
    __shared__ int pre[kStreamMaxSeq + 1];     // steps before sequence i
    __shared__ int vpre[kStreamMaxSeq + 1];    // valid sequences before sequence i
    __shared__ int lens[kStreamMaxSeq];        // seq_lens
    __shared__ int2 wtot[NW];
    __shared__ int pg[KV::kStage];             // paged: the page ids of the range's steps

    if (threadIdx.x < NW) slot_busy[threadIdx.x] = 0;
    if (threadIdx.x == 0) broken = 0;
    if (threadIdx.x < 4) cursor[threadIdx.x] = 0;
    unit_prefix<64 * NW>(seq_lens, b, S, qr.T, qr.W, g, pre, vpre, lens, wtot);  // its barriers publish the above
    // everything that steers the loops below is wave-uniform: keep it scalar
    const int T = __builtin_amdgcn_readfirstlane(pre[b]);
    const int wg = blockIdx.x;
    const int nwg = __builtin_amdgcn_readfirstlane(max(1, min((int)gridDim.x, T / kStreamMinSteps)));

    // sequences with a length out of range: NaN rows and the error flag
    // (work-group 0, one thread per sequence; such rows are rare)
    if (wg == 0) {
        const int n_row = qr.T * qr.h * D;  // out of one sequence: [T][h][d]
        for (int i = threadIdx.x; i < b; i += 64 * NW) {
            if (pre[i + 1] != pre[i]) continue;
            for (int idx = 0; idx < n_row; idx++) out[(size_t)i * n_row + idx] = __builtin_nanf("");
            if (err) atomicOr(err, MQA_DEVERR_SEQLEN);
        }
    }
    if (T == 0 || wg >= nwg) {  // uniform across the work-group
        if (threadIdx.x == 0) cut_desc[wg] = make_int4(-1, 0, 0, 0);
        return;
    }
    // a unit's allowance (in steps) for closing its segment, chosen by
    // measurement: the closes of the kernels with two blocks per wave or a
    // one-byte cache cost one to three steps' time each, those of the
    // one-block bf16 kernel under half a step (no allowance)
    constexpr int kSegC = KV::kF8 ? 4 : NHB == 2 ? (SHARED ? 6 : 3) : 0;
    const StepSplit<kSegC> split{T, nwg, g, S, qr.T, qr.W, b, pre, vpre, lens};
    int x0, x1;
    if constexpr (kSegC == 0) {
        x0 = (int)((long long)T * wg / nwg);
        x1 = (int)((long long)T * (wg + 1) / nwg);
    } else {
        // the sequences that hold the range's two ends, every thread checking
        // its share of the sequences at once
        const long long wb0 = split.wstart(wg), wb1 = split.wstart(wg + 1);
        for (int i = threadIdx.x; i < b; i += 64 * NW) {
            const long long u0 = split.useq(i), u1 = split.useq(i + 1);
            if (u0 <= wb0 && wb0 < u1) range_end[0] = split.step_in(i, wb0);
            if (u0 <= wb1 && wb1 < u1) range_end[1] = split.step_in(i, wb1);
        }
        if (threadIdx.x == 0 && wb1 >= split.useq(b)) range_end[1] = T;
        __syncthreads();
        x0 = __builtin_amdgcn_readfirstlane(range_end[0]);
        x1 = __builtin_amdgcn_readfirstlane(range_end[1]);
    }

    // paged: the page ids of both halves of the range's steps, in step order
    // (entry 2 (x - x0) + half), published by the barrier below
    const int ne = KV::kPaged ? min(2 * (x1 - x0), KV::kStage) : 0;
    if constexpr (KV::kPaged)
        stage_page_ids<64 * NW>(kv, pg, ne, [&](int e, int &i_, int &row, int &L_) {
            const int tt = x0 + (e >> 1);
            int lo = 0, hi = b;  // pre[lo] <= tt < pre[hi] (pre[b] = T > tt)
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (pre[mid] <= tt)
                    lo = mid;
                else
                    hi = mid;
            }
            i_ = lo;
            L_ = lens[lo];
            row = ((tt - pre[lo]) % seq_steps(L_, S, qr.T, qr.W) + qr.first_step(L_)) * C::STEP +
                  16 * (e & 1);
        });

    // The range's last segment [xl, x1) is claimed first, then [x0, xl): a
    // unit cut at x1 is then finished early on both sides of the cut, and
    // its merge does not fall at the end of the range. Segments are numbered
    // in claim order (sn: 0 for the last segment, then 1 + ordinal - ordinal
    // of the first, where the ordinal numbers units with steps densely: valid
    // sequences before i, times g, plus j). Record e serves the segments with
    // sn = e mod kRing one after the other, so a segment waits only for an
    // earlier-claimed one to release its record.
    for (int i = threadIdx.x; i < b; i += 64 * NW) {
        if (pre[i] <= x0 && x0 < pre[i + 1]) first_seq = i;
        if (pre[i] < x1 && x1 <= pre[i + 1]) last_seq = i;
    }
    if (threadIdx.x < 4 * kRing) {
        rec_tag[threadIdx.x / kRing][threadIdx.x % kRing] = threadIdx.x % kRing;
        rec_val[threadIdx.x / kRing][threadIdx.x % kRing] = 0;
    }
    __syncthreads();
    const int i_first = __builtin_amdgcn_readfirstlane(first_seq);
    const int i_last = __builtin_amdgcn_readfirstlane(last_seq);
    const int ord0 = __builtin_amdgcn_readfirstlane(vpre[i_first]) * g +
                     (x0 - __builtin_amdgcn_readfirstlane(pre[i_first])) /
                         seq_steps(__builtin_amdgcn_readfirstlane(lens[i_first]), S, qr.T, qr.W);
    const int n_last = seq_steps(__builtin_amdgcn_readfirstlane(lens[i_last]), S, qr.T, qr.W);
    const int p_last = __builtin_amdgcn_readfirstlane(pre[i_last]);
    const int u0_last = p_last + (x1 - 1 - p_last) / n_last * n_last;  // the last unit's first step
    const int xl = max(x0, u0_last);
    const int len_last = x1 - xl;
    // A unit cut at x1 whose first step is in this range is described for
    // streamk_combine_kernel: (sequence, K/V head, last range holding a
    // piece, slot of this range's piece).
    if (threadIdx.x == 0)
        cut_desc[wg] = (u0_last >= x0 && u0_last + n_last > x1)
                           ? make_int4(i_last, (u0_last - p_last) / n_last,
                                       split.owner(i_last, (u0_last - p_last) / n_last, n_last, n_last - 1),
                                       u0_last > x0 ? 1 : 0)
                           : make_int4(-1, 0, 0, 0);

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, qd = lane >> 4;
    // The unit's query rows are cut into blocks of 16 and the blocks into
    // ngroups groups of NHB; a wave computes all blocks of its group against
    // each step it loads, and the waves of a group share the range's steps.
    const int wph = NW / ngroups;  // waves per head group
    const int hb = w / wph, wb = w % wph;
    const int HBT = (R + C::HB - 1) / C::HB * C::HB;  // head slots per unit
    // this lane's query row in each block (padded rows reuse the last real
    // one and are never written out) and its token
    int tau[NHB];
#pragma unroll
    for (int k = 0; k < NHB; k++) tau[k] = qr.tok(min((hb * NHB + k) * C::HB + r, R - 1));

    // next step of the range for this head block, in claim order (x1: none
    // left): from the shared counter, or with det the wave's own fixed
    // sequence wb, wb + wph, ... (the same claim order, dealt round robin, so
    // that every wave always computes the same steps)
    int nclaims = 0;
    auto claim = [&]() __attribute__((always_inline)) {
        int c = 0;
        if (det) {
            c = wb + wph * nclaims++;
        } else {
            if (lane == 0) c = atomicAdd(&cursor[hb], 1);
            c = __builtin_amdgcn_readfirstlane(__shfl(c, 0));
        }
        return c >= x1 - x0 ? x1 : c < len_last ? xl + c : x0 + (c - len_last);
    };
    // unit holding flat step tt: sequence i_, its length L_ and steps n_, K/V
    // head j_, first flat step u0_ (claims move forward, but for the one jump
    // from the last segment back to x0)
    auto locate = [&](int tt, int &i_, int &L_, int &n_, int &j_, int &u0_)
                      __attribute__((always_inline)) {
        if (tt >= u0_ && tt < u0_ + n_) return;
        if (tt < u0_) i_ = i_first;
        while (__builtin_amdgcn_readfirstlane(pre[i_ + 1]) <= tt) i_++;
        L_ = __builtin_amdgcn_readfirstlane(lens[i_]);
        n_ = seq_steps(L_, S, qr.T, qr.W);
        const int p = __builtin_amdgcn_readfirstlane(pre[i_]);
        j_ = (tt - p) / n_;
        u0_ = p + j_ * n_;
    };
    auto load_q = [&](int i_, int j_, bf16x8_t (&qo)[NHB][C::KSTEPS]) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < NHB; k++)
            load_q_operand<D, F8>(q, qr.row(i_, j_, min((hb * NHB + k) * C::HB + r, R - 1)), qd,
                                  qo[k]);
    };
    // where the rows of flat step tt (of unit (i_, j_), first step u0_) are
    auto src_of = [&](int i_, int j_, int L_, int u0_, int tt, bool &bad)
                      __attribute__((always_inline)) {
        const int t0 = (tt - u0_ + qr.first_step(L_)) * C::STEP;
        if constexpr (KV::kPaged) {
            const int e = 2 * (tt - x0);
            int id0, id1;
            if (e < ne) {
                id0 = pg[e];
                id1 = pg[e + 1];
            } else {  // past what LDS holds: look the ids up
                id0 = kv.page_id(i_, t0, L_);
                id1 = kv.page_id(i_, t0 + 16, L_);
            }
            return kv.step_ids(j_, L_, t0, __builtin_amdgcn_readfirstlane(id0),
                               __builtin_amdgcn_readfirstlane(id1), bad);
        } else {
            return kv.step(i_, j_, L_, t0, bad);
        }
    };

    int t = claim();
    if (t >= x1) return;  // nothing left for this wave
    int ci = i_first, cL = 0, cn = 0, cj = 0, cu0 = 0;
    locate(t, ci, cL, cn, cj, cu0);
    bool bad_now = false;  // the current step read an invalid page
    StepData<D, F8> A, B;
    load_step<D, F8, SHARED>(src_of(ci, cj, cL, cu0, t, bad_now), lane, A);
    float cqs = F8 ? qk_base * k_scale[cj] : qk_base;  // the unit's score factor
    float cvs = F8 ? v_scale[cj] : 1.f;                // and output factor
    bf16x8_t qop[NHB][C::KSTEPS];
    load_q(ci, cj, qop);
    MfmaState<D> st[NHB];
#pragma unroll
    for (int k = 0; k < NHB; k++) st[k].reset();
    int mine = 0;  // steps of the current unit in this wave's state

    // this wave is done with the segment (range ∩ unit (ci, cj))
    auto finish_segment = [&]() __attribute__((always_inline)) {
        const int lane = opaque_lane(threadIdx.x & 63);
        const int r = lane & 15, qd = lane >> 4;
        const int seg_s = max(x0, cu0), seg_e = min(x1, cu0 + cn);
        const int sn = seg_s == xl ? 0 : __builtin_amdgcn_readfirstlane(vpre[ci]) * g + cj - ord0 + 1;
        const int e = sn & (kRing - 1);
        // rows of acc are heads 4qd+v of each block
        float Mv[NHB][4], Lv[NHB][4], l_tot[NHB];
#pragma unroll
        for (int k = 0; k < NHB; k++) {
            const float l_head = st[k].l_lane + __shfl_xor(st[k].l_lane, 16);
            l_tot[k] = l_head + __shfl_xor(l_head, 32);  // head r
#pragma unroll
            for (int v = 0; v < 4; v++) {
                Mv[k][v] = __shfl(st[k].m_ref, 4 * qd + v);
                Lv[k][v] = __shfl(l_tot[k], 4 * qd + v);
            }
        }
        if (mine == seg_e - seg_s) {  // the whole segment was this wave's: pass the record on
            lds_flag_wait(&rec_tag[hb][e], sn, &broken, err);
            if (lane == 0) lds_flag_set(&rec_tag[hb][e], sn + kRing);
        } else {  // other waves have steps of this segment
            lds_flag_wait(&slot_busy[w], 0, &broken, err);
#pragma unroll
            for (int k = 0; k < NHB; k++) {
#pragma unroll
                for (int nb = 0; nb < C::NB; nb++) slot_o[w][k][nb][lane] = st[k].acc[nb];
                if (qd == 0) slot_ml[w][k][r] = make_float2(st[k].m_ref, l_tot[k]);
            }
            if (lane == 0) slot_busy[w] = 1;
            lds_drain();
            lds_flag_wait(&rec_tag[hb][e], sn, &broken, err);  // an earlier segment may still hold the record
            const uint32_t add = ((uint32_t)mine << 8) | (1u << wb);
            uint32_t old = 0;
            if (lane == 0) old = atomicAdd(&rec_val[hb][e], add);
            const uint32_t now_ = __builtin_amdgcn_readfirstlane(__shfl(old, 0)) + add;
            if ((int)(now_ >> 8) != seg_e - seg_s) return;  // not the last: the state waits in the slot
            // the last share in: merge the others, release their slots and the
            // record. With det the merge must not depend on which wave came
            // last: it starts from an empty state and takes every parked
            // state, its own included, in wave order.
            if (lane == 0) slot_busy[w] = 0;
            uint32_t parked = now_ & 0xffu & ~(1u << wb);
            if (det) {
                parked |= 1u << wb;
#pragma unroll
                for (int k = 0; k < NHB; k++) {
#pragma unroll
                    for (int v = 0; v < 4; v++) {
                        Mv[k][v] = -INFINITY;
                        Lv[k][v] = 0.f;
                    }
#pragma unroll
                    for (int nb = 0; nb < C::NB; nb++) st[k].acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
            }
            for (uint32_t m = parked; m; m &= m - 1) {
                const int ww = hb * wph + __builtin_ctz(m);
#pragma unroll
                for (int k = 0; k < NHB; k++) {
                    float a_own[4], a_oth[4];
#pragma unroll
                    for (int v = 0; v < 4; v++) {
                        const float2 eo = slot_ml[ww][k][4 * qd + v];
                        const float Mn = fmaxf(Mv[k][v], eo.x);
                        a_own[v] = Mv[k][v] == -INFINITY ? 0.f : fast_exp2(Mv[k][v] - Mn);
                        a_oth[v] = eo.x == -INFINITY ? 0.f : fast_exp2(eo.x - Mn);
                        Lv[k][v] = fmaf(Lv[k][v], a_own[v], a_oth[v] * eo.y);
                        Mv[k][v] = Mn;
                    }
#pragma unroll
                    for (int nb = 0; nb < C::NB; nb++) {
                        const f32x4_t o = slot_o[ww][k][nb][lane];
#pragma unroll
                        for (int v = 0; v < 4; v++)
                            st[k].acc[nb][v] = fmaf(st[k].acc[nb][v], a_own[v], a_oth[v] * o[v]);
                    }
                }
                lds_drain();
                if (lane == 0) lds_flag_set(&slot_busy[ww], 0);
            }
            if (lane == 0) {
                rec_val[hb][e] = 0;
                lds_drain();
                lds_flag_set(&rec_tag[hb][e], sn + kRing);
            }
        }
        // once a wait of this work-group ran out, its rows are NaN (lds_flag_wait)
        const bool brk = __builtin_amdgcn_readfirstlane(
                             __hip_atomic_load(&broken, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) != 0;
        if (seg_s != cu0 || seg_e != cu0 + cn) {
            // a piece of a cut unit: slot 0 for the range's first segment, 1
            // for its last; streamk_combine_kernel merges the pieces
            const int slot = seg_s == x0 ? 0 : 1;
#pragma unroll
            for (int k = 0; k < NHB; k++)
#pragma unroll
                for (int v = 0; v < 4; v++) {
                    const int hs = (hb * NHB + k) * C::HB + 4 * qd + v;
                    if (hs >= R) continue;
                    const size_t prow = ((size_t)wg * 2 + slot) * HBT + hs;
#pragma unroll
                    for (int nb = 0; nb < C::NB; nb++)
                        part_o[prow * D + 16 * nb + r] = st[k].acc[nb][v] * cvs;
                    if (r == 0) part_ml[prow] = make_float2(Mv[k][v], brk ? __builtin_nanf("") : Lv[k][v]);
                }
            return;
        }
        // a whole unit: its rows, normalised
#pragma unroll
        for (int k = 0; k < NHB; k++)
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int hs = (hb * NHB + k) * C::HB + 4 * qd + v;
                if (hs >= R) continue;
                const float inv = brk ? __builtin_nanf("") : cvs / Lv[k][v];
                const size_t orow = qr.row(ci, cj, hs);
#pragma unroll
                for (int nb = 0; nb < C::NB; nb++)
                    out[orow * D + 16 * nb + r] = st[k].acc[nb][v] * inv;
            }
    };

    // one step: claim and prefetch the next, compute this one, close the
    // segment if the next claim leaves it
    auto body = [&](StepData<D, F8> &now, StepData<D, F8> &later) __attribute__((always_inline)) -> bool {
        const int t0_now = (t - cu0 + qr.first_step(cL)) * C::STEP;
        stage_v<D, F8, KV::kI8>(now, t0_now, cL, vbuf[w], lane);
        const int tn = claim();
        const bool more = tn < x1;
        int ni = ci, nL = cL, nn = cn, nj = cj, nu0 = cu0;
        if (more) locate(tn, ni, nL, nn, nj, nu0);
        const bool next_unit = more && nu0 != cu0;
        bool bad_next = false;
        // nothing left: a step that loads nothing
        load_step<D, F8, SHARED>(more ? src_of(ni, nj, nL, nu0, tn, bad_next) : kv.none(), lane,
                                 later);
        // causal ends of several tokens: this lane's row in each block, the
        // wave's earliest
        // (and the window starts)
        int t_row[NHB], t_rs[NHB];
#pragma unroll
        for (int k = 0; k < NHB; k++) {
            t_row[k] = cL - qr.T + 1 + tau[k];
            t_rs[k] = qr.W > 0 ? max(0, t_row[k] - qr.W) : 0;
        }
        const int t_hs = qr.W > 0 ? max(0, cL - qr.W) : 0;
        compute_step<D, MULTI, NHB, F8, KV::kI8>(now, t0_now, cL, cL - qr.T + 1, t_row, t_hs, t_rs,
                                                 qop, st, vbuf[w], lane, cqs);
        if (bad_now) poison_state<D>(st, err, lane);
        bad_now = bad_next;
        mine++;
        // the next unit's q, in flight during the segment's close
        if (next_unit) load_q(ni, nj, qop);
        float nqs = cqs, nvs = cvs;  // the next unit's factors, in flight with its q
        if (F8 && next_unit) {
            nqs = qk_base * k_scale[nj];
            nvs = v_scale[nj];
        }
        if (!more || next_unit) {
            finish_segment();
#pragma unroll
            for (int k = 0; k < NHB; k++) st[k].reset();
            mine = 0;
        }
        cqs = nqs;
        cvs = nvs;
        if (!more) return false;
        // wave-uniform; said explicitly so that the loop state stays scalar
        t = __builtin_amdgcn_readfirstlane(tn);
        ci = __builtin_amdgcn_readfirstlane(ni);
        cL = __builtin_amdgcn_readfirstlane(nL);
        cn = __builtin_amdgcn_readfirstlane(nn);
        cj = __builtin_amdgcn_readfirstlane(nj);
        cu0 = __builtin_amdgcn_readfirstlane(nu0);
        return true;
    };
    while (body(A, B) && body(B, A)) {
    }
}

// Units cut between ranges, after streamk_mfma_kernel: block (w, y) merges
// head slots HPB*y .. HPB*y+HPB-1 of the unit described by cut_desc[w] (the
// first range's piece in its slot cut_desc[w].w, the following ranges'
// pieces in slot 0) and writes those rows of `out`. Threads are (head slot,
// piece lane, four columns); piece lane k merges pieces w+k, w+k+PL, ...
// (four loads in flight at a time) and the lanes are merged in order through
// LDS, so the result is the same every call. Many head slots per block suit
// units cut into few pieces, many piece lanes units cut into many.
template <int D, int HPB>
__global__ void __launch_bounds__(256)
streamk_combine_kernel(const float *__restrict__ part_o, const float2 *__restrict__ part_ml,
                       const int4 *__restrict__ cut_desc, const QRows<true> qr, int R, int HBT,
                       float *__restrict__ out) {
    constexpr int C4 = D / 4;               // float4 columns per row
    constexpr int PL = 256 / (HPB * C4);    // piece lanes per head slot
    constexpr int BATCH = 4;
    static_assert(PL >= 1 && HPB * PL * C4 == 256, "block shape");
    __shared__ f32x4_t s_num[HPB][PL][C4];
    __shared__ float2 s_md[HPB][PL][C4];
    const int wf = blockIdx.x;
    const int4 dsc = cut_desc[wf];
    if (dsc.x < 0) return;  // uniform over the block
    const int wl = dsc.z, slot_f = dsc.w;
    const int hh = threadIdx.x / (PL * C4), pl = (threadIdx.x / C4) % PL, c4 = threadIdx.x % C4;
    const int hs = blockIdx.y * HPB + hh;
    const bool live_row = hs < R;
    float M = -INFINITY, den = 0.f;
    f32x4_t num = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int p0 = wf + pl; live_row && p0 <= wl; p0 += BATCH * PL) {
        float2 e[BATCH];
        f32x4_t o[BATCH];
#pragma unroll
        for (int k = 0; k < BATCH; k++) {
            const int p = p0 + k * PL;
            const size_t prow = ((size_t)p * 2 + (p == wf ? slot_f : 0)) * HBT + hs;
            const bool live = p <= wl;
            e[k] = live ? part_ml[prow] : make_float2(-INFINITY, 0.f);
            o[k] = live ? *(const f32x4_t *)(part_o + prow * D + 4 * c4) : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        float Mb = M;
#pragma unroll
        for (int k = 0; k < BATCH; k++) Mb = fmaxf(Mb, e[k].x);
        const float rs = M == -INFINITY ? 0.f : fast_exp2(M - Mb);
        num *= rs;
        den *= rs;
        M = Mb;
#pragma unroll
        for (int k = 0; k < BATCH; k++) {
            const float wgt = e[k].x == -INFINITY ? 0.f : fast_exp2(e[k].x - M);
            num += wgt * o[k];
            den = fmaf(wgt, e[k].y, den);
        }
    }
    if (PL > 1) {
        s_num[hh][pl][c4] = num;
        s_md[hh][pl][c4] = make_float2(M, den);
        __syncthreads();
        if (pl != 0) return;
        for (int k = 1; k < PL; k++) {
            const float2 md = s_md[hh][k][c4];
            const float Mn = fmaxf(M, md.x);
            const float a0 = M == -INFINITY ? 0.f : fast_exp2(M - Mn);
            const float a1 = md.x == -INFINITY ? 0.f : fast_exp2(md.x - Mn);
            num = num * a0 + a1 * s_num[hh][k][c4];
            den = den * a0 + a1 * md.y;
            M = Mn;
        }
    }
    if (!live_row) return;
    const size_t row = qr.row(dsc.x, dsc.y, hs);
    *(f32x4_t *)(out + row * D + 4 * c4) = num * (1.f / den);
}

// ---------------------------------------------------------------------------
// combine: out = sum_s 2^(m_s-M) o_s / sum_s 2^(m_s-M) l_s over live partitions
// ---------------------------------------------------------------------------

// Block (k, i): partial row i*T*h + k (k = j*R + rho: K/V head j, query row
// rho of the unit), written to out row qr.row(i, j, rho). Threads are (piece
// lane, four columns); piece lane pl merges partitions pl, pl+PL, ... (BATCH
// loads in flight at a time) and the lanes are merged in order through LDS,
// so the result is the same every call. The first batch is loaded before the
// sequence length arrives (partitions below nsplit lie in the workspace
// whatever the length) and masked once the sequence's partition count is
// known, which saves one dependent round trip to memory.
template <int D, int BATCH>
__global__ void __launch_bounds__(256)
combine_kernel(const float *__restrict__ part_o, const float2 *__restrict__ part_ml,
               const int32_t *__restrict__ seq_lens, const QRows<true> qr, int R, int S, int chunk,
               int nsplit, float *__restrict__ out, int32_t *__restrict__ err) {
    constexpr int C4 = D / 4;           // float4 columns per row
    constexpr int PL = 256 / C4;        // piece lanes
    __shared__ f32x4_t s_num[PL][C4];
    __shared__ float2 s_md[PL][C4];
    const int k = blockIdx.x, i = blockIdx.y;
    const int pl = threadIdx.x / C4, c4 = threadIdx.x % C4;
    const size_t row = (size_t)i * qr.T * qr.h + k;
    const size_t orow = qr.row(i, k / R, k % R);
    const float2 *ml = part_ml + row * nsplit;
    const float *po = part_o + row * nsplit * D + 4 * c4;
    float2 e[BATCH];
    f32x4_t o[BATCH];
#pragma unroll
    for (int kk = 0; kk < BATCH; kk++) {
        const int p = pl + kk * PL;
        const bool ok = p < nsplit;
        e[kk] = ok ? ml[p] : make_float2(-INFINITY, 0.f);
        o[kk] = ok ? *(const f32x4_t *)(po + (size_t)p * D) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const int L = seq_lens[i];
    if (L < qr.T || L > S) {  // uniform over the block
        if (pl == 0) *(f32x4_t *)(out + orow * D + 4 * c4) = f32x4_t{1.f, 1.f, 1.f, 1.f} * __builtin_nanf("");
        if (k == 0 && threadIdx.x == 0 && err) atomicOr(err, MQA_DEVERR_SEQLEN);
        return;
    }
    // partitions start at the window's first step (0 without a window)
    const int n = (L - window_first_step(L, qr.T, qr.W) * 32 + chunk - 1) / chunk;
    float M = -INFINITY, den = 0.f;
    f32x4_t num = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int p0 = pl; p0 < n; p0 += BATCH * PL) {
        if (p0 != pl) {
#pragma unroll
            for (int kk = 0; kk < BATCH; kk++) {
                const int p = p0 + kk * PL;
                const bool ok = p < n;
                e[kk] = ok ? ml[p] : make_float2(-INFINITY, 0.f);
                o[kk] = ok ? *(const f32x4_t *)(po + (size_t)p * D) : f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
        } else {  // the first batch: drop partitions past the sequence's last
#pragma unroll
            for (int kk = 0; kk < BATCH; kk++)
                if (p0 + kk * PL >= n) {
                    e[kk] = make_float2(-INFINITY, 0.f);
                    o[kk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
        }
        float Mb = M;
#pragma unroll
        for (int kk = 0; kk < BATCH; kk++) Mb = fmaxf(Mb, e[kk].x);
        const float rs = M == -INFINITY ? 0.f : fast_exp2(M - Mb);
        num *= rs;
        den *= rs;
        M = Mb;
#pragma unroll
        for (int kk = 0; kk < BATCH; kk++) {
            const float wgt = e[kk].x == -INFINITY ? 0.f : fast_exp2(e[kk].x - M);
            num += wgt * o[kk];
            den = fmaf(wgt, e[kk].y, den);
        }
    }
    s_num[pl][c4] = num;
    s_md[pl][c4] = make_float2(M, den);
    __syncthreads();
    if (pl != 0) return;
    for (int kk = 1; kk < PL; kk++) {
        const float2 md = s_md[kk][c4];
        const float Mn = fmaxf(M, md.x);
        const float a0 = M == -INFINITY ? 0.f : fast_exp2(M - Mn);
        const float a1 = md.x == -INFINITY ? 0.f : fast_exp2(md.x - Mn);
        num = num * a0 + a1 * s_num[kk][c4];
        den = den * a0 + a1 * md.y;
        M = Mn;
    }
    *(f32x4_t *)(out + orow * D + 4 * c4) = num * (1.f / den);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

// Launch a kernel and return the launch's own status (the runtime's last-error
// slot may hold an unrelated error left by the caller's earlier calls). The
// arguments are converted to the kernel's parameter types and passed by address,
// as hipLaunchKernel copies them at the call.
template <typename... P, typename... A>
hipError_t klaunch(void (*k)(P...), dim3 grid, dim3 block, hipStream_t stream, A &&...a) {
    std::tuple<std::decay_t<P>...> args(std::forward<A>(a)...);
    return std::apply(
        [&](auto &...x) {
            void *ptrs[] = {(void *)&x...};
            return hipLaunchKernel((const void *)k, grid, block, ptrs, 0, stream);
        },
        args);
}
#define MQA_LAUNCH(...)                                          \
    do {                                                          \
        if (klaunch(__VA_ARGS__) != hipSuccess) return MQA_ERR_HIP; \
    } while (0)

// The log-sum-exp combine over nsplit partitions per row: eight loads in
// flight per piece lane when a lane has more than four partitions to merge
// (one round trip instead of two), four otherwise.
template <int D>
mqa_status launch_combine(dim3 grid, hipStream_t stream, const float *part_o, const float2 *part_ml,
                    const int32_t *seq_lens, const QRows<true> &qc, int R, int S, int chunk,
                    int nsplit, float *out, int32_t *err_flags) {
    constexpr int PL = 256 / (D / 4);
    if ((nsplit + PL - 1) / PL > 4)
        MQA_LAUNCH(combine_kernel<D, 8>, grid, dim3(256), stream, part_o, part_ml, seq_lens, qc, R, S, chunk, nsplit, out, err_flags);
    else
        MQA_LAUNCH(combine_kernel<D, 4>, grid, dim3(256), stream, part_o, part_ml, seq_lens, qc, R, S, chunk, nsplit, out, err_flags);
    return MQA_OK;
}

constexpr float kLog2e = 1.4426950408889634f;
// Compute units the schedules are planned for: the 256 of a gfx950 part
// (MI355X, MI350X). A constant, so that the host-side queries (partition
// length, workspace size, schedule) are pure functions of their arguments and
// never touch the HIP runtime or depend on which device is current; on a
// device with fewer compute units the extra work-groups simply queue.
constexpr int kPlanCUs = 256;

int heads_per_wg(int G) {
    int hpw = 1;
    while (hpw < G && hpw < 8) hpw <<= 1;
    return hpw;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

mqa_status check_sizes(int b, int h, int g, int S, int d, mqa_dtype dt, int split_chunk) {
    if (b < 1 || h < 1 || g < 1 || S < 1 || d < 1) return MQA_ERR_SHAPE;
    if (h % g != 0) return MQA_ERR_SHAPE;  // [GQA notes] §四, §十 (divisibility)
    if (b > 65535 || (long long)g * h > (1ll << 30)) return MQA_ERR_SHAPE;
    if (d != 64 && d != 128) return MQA_ERR_UNSUPPORTED;
    if (dt != MQA_F32 && dt != MQA_BF16) return MQA_ERR_UNSUPPORTED;
    if (split_chunk < 0 || split_chunk % kTile != 0) return MQA_ERR_UNSUPPORTED;
    // one K/V head's S rows stay below 2 GiB: kernels address them with 32-bit offsets
    if ((long long)S * d * (dt == MQA_BF16 ? 2 : 4) >= (1ll << 31)) return MQA_ERR_SHAPE;
    return MQA_OK;
}

// Query heads one work-group scores: bf16 runs on the matrix cores in blocks
// of 16 heads, fp32 on the vector ALUs in blocks of up to 8.
int wg_heads(mqa_dtype dt, int G) { return dt == MQA_BF16 ? 16 : heads_per_wg(G); }

// Automatic partition length: about one work-group per compute unit (each
// work-group's waves then stream tens of steps; measured best for MQA at
// 32K context, the 32-layer sweeps and short contexts alike — more, shorter
// partitions only add start-up latency and combine work).
// Query rows R of a (sequence, K/V head) unit on the matrix cores: blocks of
// 16 rows; a wave computes blk_per_wave (NHB) blocks against each K/V step
// it loads (two once there is more than one: the K/V registers then serve
// 32 rows), and the unit's blocks form `groups` such groups.
struct RowBlocks {
    int blocks, per_wave, groups;
};
RowBlocks row_blocks(int R) {
    RowBlocks rb;
    rb.blocks = (R + 15) / 16;
    rb.per_wave = rb.blocks > 1 ? 2 : 1;
    rb.groups = (rb.blocks + rb.per_wave - 1) / rb.per_wave;
    return rb;
}

// Positions a call's partitions cover at most: the capacity, or with a
// sliding window of W positions and T tokens the span from the window's
// first 32-position step to the end (L - 32*floor((L-T+1-W)/32) <= W+T+30).
int window_span(int S, int T, int W) {
    const long long span = (long long)W + T + 30;
    return W > 0 && span < S ? (int)span : S;
}

// (T query tokens: T*h/g query rows per (sequence, K/V head).)
int resolve_chunk(int b, int h, int g, int S, mqa_dtype dt, int split_chunk, int T = 1) {
    if (split_chunk > 0) return split_chunk;
    const int G = T * (h / g);
    const long long groups = (long long)b * g *
        (dt == MQA_BF16 ? row_blocks(G).groups : (G + wg_heads(dt, G) - 1) / wg_heads(dt, G));
    const long long want = (kPlanCUs + groups - 1) / groups;  // partitions per group
    long long c = ((long long)S + want - 1) / want;
    c = (c + kTile - 1) / kTile * kTile;
    const long long cap = ((long long)S + kTile - 1) / kTile * kTile;
    if (c > cap) c = cap;
    return (int)c;
}

size_t workspace_for(int b, int h, int S, int d, int chunk) {
    const size_t nsplit = ((size_t)S + chunk - 1) / chunk;
    const size_t rows = (size_t)b * h * nsplit;
    const size_t o_bytes = (rows * d * sizeof(float) + 255) & ~(size_t)255;
    return o_bytes + rows * sizeof(float2);
}

// The balanced schedule serves bf16 calls with automatic partitioning, up to
// kStreamMaxSeq sequences and 64 query heads per K/V head.
// It pays where there are many units (sequence, K/V head) whose lengths
// differ; with few units every unit would be cut into many pieces and the
// fixed partitions (merged in parallel by combine_kernel) do better.
bool use_streamk(int b, int h, int g, int S, mqa_dtype dt, int split_chunk, mqa_kernel kernel,
                 int T = 1) {
    const int ngr = row_blocks(T * (h / g)).groups;
    const long long units = (long long)b * g;
    if (units * ((S + 31) / 32) >= (1ll << 31)) return false;  // step indices are 32-bit
    return dt == MQA_BF16 && kernel != MQA_KERNEL_VALU && split_chunk == 0 &&
           b <= kStreamMaxSeq && units >= kStreamMinUnits &&
           (ngr == 1 || ngr == 2 || ngr == 4);
}

// Balanced-schedule workspace: [partials o][partials (m, l)][cut-unit
// descriptors], each part 256-byte aligned; two pieces per work-group.
struct StreamkLayout {
    size_t o_bytes, ml_off, desc_off, total;
};
StreamkLayout streamk_layout(int h, int g, int d, int T = 1) {
    const size_t hbt = (size_t)((T * (h / g) + 15) / 16) * 16;
    const size_t rows = (size_t)kStreamMaxWG * 2 * hbt;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    StreamkLayout L;
    L.o_bytes = up(rows * d * sizeof(float));
    L.ml_off = L.o_bytes;
    L.desc_off = L.ml_off + up(rows * sizeof(float2));
    L.total = L.desc_off + kStreamMaxWG * sizeof(int4);
    return L;
}

// Workspace bytes: the larger of the two paths' needs (the same workspace
// serves every kernel choice)
size_t workspace_need(int b, int h, int g, int S, int d, mqa_dtype dt, int split_chunk,
                      mqa_kernel kernel, int T = 1) {
    size_t need = workspace_for(b, T * h, S, d, resolve_chunk(b, h, g, S, dt, split_chunk, T));
    if (use_streamk(b, h, g, S, dt, split_chunk, kernel, T)) {
        const size_t sk = streamk_layout(h, g, d, T).total;
        if (sk > need) need = sk;
    }
    return need;
}

// Work-groups of the balanced schedule: one per compute unit (the kernel
// uses fewer when the call has fewer than kStreamMinSteps steps for each).
int streamk_wgs(int b, int g, int S) {
    const int cus = kPlanCUs;
    const long long tmax = (long long)b * g * ((S + 31) / 32);
    long long n = (tmax + kStreamMinSteps - 1) / kStreamMinSteps;
    if (n > cus) n = cus;
    if (n > kStreamMaxWG) n = kStreamMaxWG;
    if (n < 1) n = 1;
    return (int)n;
}

template <typename T, int D, int HPW>
mqa_status launch_rows(const void *q, const void *k, const void *v, const int32_t *seq_lens, int b,
                 int h, int g, int S, float qk_scale_log2, int chunk, int nsplit, float *part_o,
                 float2 *part_ml, hipStream_t stream) {
    const int G = h / g;
    const int nhc = (G + HPW - 1) / HPW;
    dim3 grid(nsplit, g * nhc, b);
    MQA_LAUNCH(split_rows_kernel<T, D, HPW>, grid, dim3(64 * HPW), stream, (const T *)q, (const T *)k, (const T *)v, seq_lens, h, g, S, G, nhc, chunk, nsplit, qk_scale_log2, part_o, part_ml);
    return MQA_OK;
}

template <typename T, int D>
mqa_status dispatch_rows(int hpw, const void *q, const void *k, const void *v, const int32_t *seq_lens,
                   int b, int h, int g, int S, float qs, int chunk, int nsplit, float *po,
                   float2 *pml, hipStream_t st) {
    switch (hpw) {
        case 1: return launch_rows<T, D, 1>(q, k, v, seq_lens, b, h, g, S, qs, chunk, nsplit, po, pml, st);
        case 2: return launch_rows<T, D, 2>(q, k, v, seq_lens, b, h, g, S, qs, chunk, nsplit, po, pml, st);
        case 4: return launch_rows<T, D, 4>(q, k, v, seq_lens, b, h, g, S, qs, chunk, nsplit, po, pml, st);
        default: return launch_rows<T, D, 8>(q, k, v, seq_lens, b, h, g, S, qs, chunk, nsplit, po, pml, st);
    }
}

// The matrix-core paths (bf16) for one K/V source: the balanced schedule
// (+ its cut-unit merge) or fixed partitions (+ the log-sum-exp combine).
// T query tokens per sequence (T > 1: the causal variant of the kernels).
template <int D, class KV, bool MULTI, int NHB>
mqa_status run_mfma_rows(const KV &kv, const void *q, const int32_t *seq_lens, int b, int T,
                         int h, int g, int S, float qs, const float *k_scale,
                         const float *v_scale, float *out, void *workspace, int chunk,
                         int nsplit, bool balanced, int32_t *err_flags, hipStream_t stream,
                         int W, int det = 0) {
    const int Gh = h / g, R = T * Gh;
    const int nhb = (R + 15) / 16;
    const int ngroups = (nhb + NHB - 1) / NHB;
    const QRows<MULTI> qr{T, Gh, h, W};
    const QRows<true> qc{T, Gh, h, W};
    if (balanced) {
        const int nwg = streamk_wgs(b, g, window_span(S, T, W));
        const StreamkLayout L = streamk_layout(h, g, D, T);
        float *po = (float *)workspace;
        float2 *pml = (float2 *)((uint8_t *)workspace + L.ml_off);
        int4 *desc = (int4 *)((uint8_t *)workspace + L.desc_off);
        // a code cache (fp8, int8) costs more per byte (the decode to bf16): eight waves
        // per compute unit then hide the latencies of one another's steps
        // (measured faster for fp8, slower for bf16, whose steps are cheaper)
        constexpr int NWV = (KV::kF8 && NHB == 1) ? 8 : kStreamWaves;
        // several head groups read each step one after another: cached loads,
        // so that the later groups find it in L2 (streamed, about half of
        // their reads went to HBM again: 956 MB fetched per call for 643 MB
        // with eight tokens on gqa-70b)
        if (ngroups > 1)
            MQA_LAUNCH(streamk_mfma_kernel<D, NWV, KV, MULTI, NHB, true>, dim3(nwg), dim3(64 * NWV), stream, (const uint16_t *)q, kv, seq_lens, b, qr, g, S, R, ngroups, qs, k_scale, v_scale, out, po, pml, desc, err_flags, det);
        else
            MQA_LAUNCH(streamk_mfma_kernel<D, NWV, KV, MULTI, NHB>, dim3(nwg), dim3(64 * NWV), stream, (const uint16_t *)q, kv, seq_lens, b, qr, g, S, R, ngroups, qs, k_scale, v_scale, out, po, pml, desc, err_flags, det);
        // pieces per cut unit: ~2 when there are more units than work-groups,
        // ~nwg/units when each unit spans many ranges
        constexpr int HPB = 256 / (D / 4);  // head slots per block with one piece lane
        if ((long long)b * g * 4 < nwg)
            MQA_LAUNCH(streamk_combine_kernel<D, 1>, dim3(nwg, R), dim3(256), stream, po, pml, desc, qc, R, nhb * 16, out);
        else
            MQA_LAUNCH(streamk_combine_kernel<D, HPB>, dim3(nwg, (R + HPB - 1) / HPB), dim3(256), stream, po, pml, desc, qc, R, nhb * 16, out);
        return MQA_OK;
    }
    const size_t rows = (size_t)b * T * h * nsplit;
    float *part_o = (float *)workspace;
    float2 *part_ml =
        (float2 *)((uint8_t *)workspace + ((rows * D * sizeof(float) + 255) & ~(size_t)255));
    // more than two blocks of rows (several tokens of many heads): work-groups
    // of eight waves sharing each step through LDS, one block per wave
    // (measured: MQA 32K with four tokens 71 -> 55 us); up to two blocks, one
    // wave computes both (its partitions hold few steps per wave, where the
    // pair kernel's per-step barrier costs more than its second wave gains)
    if (nhb > 2) {
        const int ng2 = (nhb + 1) / 2;
        MQA_LAUNCH(split_pair_kernel<D, KV, MULTI>, dim3(nsplit, g * ng2, b), dim3(512), stream, (const uint16_t *)q, kv, seq_lens, qr, g, S, R, ng2, chunk, nsplit, qs, k_scale, v_scale, part_o, part_ml, err_flags);
    } else {
        MQA_LAUNCH(split_mfma_kernel<D, KV, MULTI, NHB>, dim3(nsplit, g * ngroups, b), dim3(256), stream, (const uint16_t *)q, kv, seq_lens, qr, g, S, R, ngroups, chunk, nsplit, qs, k_scale, v_scale, part_o, part_ml, err_flags);
    }
    return launch_combine<D>(dim3(T * h, b), stream, part_o, part_ml, seq_lens, qc, R, S, chunk,
                             nsplit, out, err_flags);
}

// (several tokens or a sliding window: the MULTI kernels, with per-row
// ends and starts)
template <int D, class KV>
mqa_status run_mfma(const KV &kv, const void *q, const int32_t *seq_lens, int b, int T, int h,
                    int g, int S, float qs, float *out, void *workspace, int chunk, int nsplit,
                    bool balanced, int32_t *err_flags, hipStream_t stream,
                    const float *k_scale = nullptr, const float *v_scale = nullptr, int W = 0,
                    int det = 0) {
    const RowBlocks rb = row_blocks(T * (h / g));
    // one-byte codes, balanced schedule, two blocks: one block per wave in
    // eight waves (two head groups reading each step, the second from L2)
    // rather than both blocks in each of four waves
    const bool two = rb.per_wave == 2 && !(KV::kF8 && balanced && rb.blocks == 2);
    if (T > 1 || W > 0) {
        if (two)
            return run_mfma_rows<D, KV, true, 2>(kv, q, seq_lens, b, T, h, g, S, qs, k_scale,
                                                 v_scale, out, workspace, chunk, nsplit, balanced,
                                                 err_flags, stream, W, det);
        return run_mfma_rows<D, KV, true, 1>(kv, q, seq_lens, b, T, h, g, S, qs, k_scale, v_scale,
                                             out, workspace, chunk, nsplit, balanced, err_flags,
                                             stream, W, det);
    }
    if (two)
        return run_mfma_rows<D, KV, false, 2>(kv, q, seq_lens, b, 1, h, g, S, qs, k_scale, v_scale,
                                              out, workspace, chunk, nsplit, balanced, err_flags,
                                              stream, 0, det);
    return run_mfma_rows<D, KV, false, 1>(kv, q, seq_lens, b, 1, h, g, S, qs, k_scale, v_scale, out,
                                          workspace, chunk, nsplit, balanced, err_flags, stream, 0,
                                          det);
}

// T-token calls: T in [1, S]; beyond one token only the bf16 matrix-core path
mqa_status check_tokens(int T, int h, int S, mqa_dtype dt) {
    if (T < 1 || T > S || (T > 1 && (long long)T * h > (1ll << 24))) return MQA_ERR_SHAPE;
    if (T > 1 && dt != MQA_BF16) return MQA_ERR_UNSUPPORTED;
    return MQA_OK;
}

// ---- the scratch of the no-allocation entry point ----

// Partials of mqa_decode_attn_noalloc, in device memory the library owns: a
// file-scope array, one copy on each GPU the library runs on (held until the
// process ends). Its size bounds the calls that entry point takes.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// The device address of the current device's copy. Host code must not pass
// `scratch` itself to a kernel (on the host it names a stand-in, not device
// memory): its address is looked up once per device, with that device
// current, on the first call there, and kept.
constexpr int kMaxDevices = 64;
void *g_scratch[kMaxDevices];
hipError_t g_scratch_rc[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

mqa_status scratch_of_current_device(void **ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MQA_ERR_HIP;
    std::call_once(g_scratch_once[dev], [dev] {
        void *p = nullptr;
        g_scratch_rc[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch[dev] = p;
    });
    if (g_scratch_rc[dev] != hipSuccess || !g_scratch[dev]) return MQA_ERR_HIP;
    *ptr = g_scratch[dev];
    return MQA_OK;
}

}  // namespace

extern "C" {

const char *mqa_status_string(mqa_status s) {
    switch (s) {
        case MQA_OK: return "ok";
        case MQA_ERR_NULL: return "a required pointer is NULL";
        case MQA_ERR_SHAPE: return "invalid sizes (a size < 1, or h not a multiple of g)";
        case MQA_ERR_UNSUPPORTED: return "unsupported head dim, dtype or split_chunk";
        case MQA_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
        case MQA_ERR_WORKSPACE: return "workspace missing or too small";
        case MQA_ERR_HIP: return "HIP launch error";
        case MQA_ERR_SCRATCH:
            return "the call needs more scratch than mqa_decode_attn_noalloc holds (64 MiB)";
        default: break;
    }
    return "unknown status";
}

uint64_t mqa_kv_bytes(int layers, int g, int64_t S, int d, int dtype_bytes) {
    if (layers < 0 || g < 0 || S < 0 || d < 0 || dtype_bytes < 0) return 0;
    return 2ull * (uint64_t)layers * (uint64_t)g * (uint64_t)S * (uint64_t)d * (uint64_t)dtype_bytes;
}

int mqa_decode_schedule(int b, int h, int g, int S, int d, mqa_dtype dt, int split_chunk,
                        mqa_kernel kernel) {
    if (check_sizes(b, h, g, S, d, dt, split_chunk) != MQA_OK) return -1;
    if (kernel != MQA_KERNEL_AUTO && kernel != MQA_KERNEL_VALU && kernel != MQA_KERNEL_MFMA &&
        kernel != MQA_KERNEL_MFMA_DETERMINISTIC)
        return -1;
    if ((kernel == MQA_KERNEL_MFMA || kernel == MQA_KERNEL_MFMA_DETERMINISTIC) && dt != MQA_BF16) return -1;
    if (use_streamk(b, h, g, S, dt, split_chunk, kernel)) return MQA_SCHEDULE_MFMA_BALANCED;
    return (dt == MQA_BF16 && kernel != MQA_KERNEL_VALU) ? MQA_SCHEDULE_MFMA_PARTITIONS
                                                         : MQA_SCHEDULE_VALU_PARTITIONS;
}

int mqa_decode_resolve_chunk(int b, int h, int g, int S, int d, mqa_dtype dt, int split_chunk) {
    if (check_sizes(b, h, g, S, d, dt, split_chunk) != MQA_OK) return -1;
    return resolve_chunk(b, h, g, S, dt, split_chunk);
}

size_t mqa_decode_workspace_bytes(int b, int h, int g, int S, int d, mqa_dtype dt,
                                  int split_chunk) {
    if (check_sizes(b, h, g, S, d, dt, split_chunk) != MQA_OK) return 0;
    // enough for every kernel choice of mqa_decode_attn_kernel
    return workspace_need(b, h, g, S, d, dt, split_chunk, MQA_KERNEL_AUTO);
}

mqa_status mqa_append_kv_multi(void *k_cache, void *v_cache, const void *k_new,
                               const void *v_new, const int32_t *seq_lens, int b, int T, int g,
                               int S, int d, mqa_dtype dt, int32_t *err_flags, hipStream_t stream) {
    if (!k_cache || !v_cache || !k_new || !v_new || !seq_lens) return MQA_ERR_NULL;
    mqa_status st = check_sizes(b, g, g, S, d, dt, 0);
    if (st != MQA_OK) return st;
    if (T < 1 || T > S) return MQA_ERR_SHAPE;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
        return MQA_ERR_ALIGN;
    const int row_bytes = d * (dt == MQA_BF16 ? 2 : 4);
    const long long total = 2ll * b * T * g * (row_bytes / 16);
    const int threads = 256;
    const long long blocks = (total + threads - 1) / threads;
    if (blocks > 0x7fffffffll) return MQA_ERR_SHAPE;
    MQA_LAUNCH(append_kv_kernel, dim3((unsigned)blocks), dim3(threads), stream, (uint8_t *)k_cache, (uint8_t *)v_cache, (const uint8_t *)k_new, (const uint8_t *)v_new, seq_lens, b, T, g, S, row_bytes, err_flags);
    return MQA_OK;
}

mqa_status mqa_append_kv(void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                         const int32_t *seq_lens, int b, int g, int S, int d, mqa_dtype dt,
                         int32_t *err_flags, hipStream_t stream) {
    return mqa_append_kv_multi(k_cache, v_cache, k_new, v_new, seq_lens, b, 1, g, S, d, dt,
                               err_flags, stream);
}

mqa_status mqa_decode_attn_kernel(const void *q, const void *k_cache, const void *v_cache,
                                  const int32_t *seq_lens, int b, int h, int g, int S, int d,
                                  mqa_dtype dt, float scale, float *out, void *workspace,
                                  size_t workspace_bytes, int split_chunk, int32_t *err_flags,
                                  mqa_kernel kernel, hipStream_t stream) {
    if (!q || !k_cache || !v_cache || !seq_lens || !out) return MQA_ERR_NULL;
    mqa_status st = check_sizes(b, h, g, S, d, dt, split_chunk);
    if (st != MQA_OK) return st;
    if (kernel != MQA_KERNEL_AUTO && kernel != MQA_KERNEL_VALU && kernel != MQA_KERNEL_MFMA &&
        kernel != MQA_KERNEL_MFMA_DETERMINISTIC)
        return MQA_ERR_UNSUPPORTED;
    if ((kernel == MQA_KERNEL_MFMA || kernel == MQA_KERNEL_MFMA_DETERMINISTIC) && dt != MQA_BF16)
        return MQA_ERR_UNSUPPORTED;
    const bool use_mfma = dt == MQA_BF16 && kernel != MQA_KERNEL_VALU;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return MQA_ERR_ALIGN;
    const int chunk = resolve_chunk(b, h, g, S, dt, split_chunk);
    const int nsplit = (S + chunk - 1) / chunk;
    const size_t need = workspace_need(b, h, g, S, d, dt, split_chunk, kernel);
    if (!workspace || workspace_bytes < need) return MQA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MQA_ERR_ALIGN;
    const float qs = scale * kLog2e;

    const size_t rows = (size_t)b * h * nsplit;
    uint8_t *wsp = (uint8_t *)workspace;
    float *part_o = (float *)wsp;
    float2 *part_ml = (float2 *)(wsp + ((rows * d * sizeof(float) + 255) & ~(size_t)255));
    const int hpw = heads_per_wg(h / g);

    if (use_mfma) {
        const bool bal = use_streamk(b, h, g, S, dt, split_chunk, kernel);
        const uint8_t *kb = (const uint8_t *)k_cache, *vb = (const uint8_t *)v_cache;
        const int det = kernel == MQA_KERNEL_MFMA_DETERMINISTIC;
        if (d == 128)
            return run_mfma<128>(ContigKV<128>{kb, vb, g, S}, q, seq_lens, b, 1, h, g, S, qs, out,
                                 workspace, chunk, nsplit, bal, err_flags, stream, nullptr, nullptr,
                                 0, det);
        return run_mfma<64>(ContigKV<64>{kb, vb, g, S}, q, seq_lens, b, 1, h, g, S, qs, out,
                            workspace, chunk, nsplit, bal, err_flags, stream, nullptr, nullptr, 0,
                            det);
    }
    if (dt == MQA_BF16)
        st = d == 128 ? dispatch_rows<uint16_t, 128>(hpw, q, k_cache, v_cache, seq_lens, b, h, g, S, qs, chunk, nsplit, part_o, part_ml, stream)
                      : dispatch_rows<uint16_t, 64>(hpw, q, k_cache, v_cache, seq_lens, b, h, g, S, qs, chunk, nsplit, part_o, part_ml, stream);
    else  // fp32 rows of 128 elements need at least two waves per work-group
        st = d == 128 ? dispatch_rows<float, 128>(hpw < 2 ? 2 : hpw, q, k_cache, v_cache, seq_lens, b, h, g, S, qs, chunk, nsplit, part_o, part_ml, stream)
                      : dispatch_rows<float, 64>(hpw, q, k_cache, v_cache, seq_lens, b, h, g, S, qs, chunk, nsplit, part_o, part_ml, stream);
    if (st != MQA_OK) return st;
    const QRows<true> qc{1, h / g, h, 0};
    if (d == 128)
        return launch_combine<128>(dim3(h, b), stream, part_o, part_ml, seq_lens, qc, h / g, S,
                                   chunk, nsplit, out, err_flags);
    return launch_combine<64>(dim3(h, b), stream, part_o, part_ml, seq_lens, qc, h / g, S, chunk,
                              nsplit, out, err_flags);
}

mqa_status mqa_decode_attn(const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *seq_lens, int b, int h, int g, int S, int d,
                           mqa_dtype dt, float scale, float *out, void *workspace,
                           size_t workspace_bytes, int split_chunk, int32_t *err_flags,
                           hipStream_t stream) {
    return mqa_decode_attn_kernel(q, k_cache, v_cache, seq_lens, b, h, g, S, d, dt, scale, out,
                                  workspace, workspace_bytes, split_chunk, err_flags,
                                  MQA_KERNEL_AUTO, stream);
}

mqa_status mqa_decode_attn_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                   const int32_t *seq_lens, int b, int h, int g, int S, int d,
                                   mqa_dtype dt, float scale, float *out, int split_chunk,
                                   int32_t *err_flags, hipStream_t stream) {
    // host-detectable errors first, then the size against the scratch array
    if (!q || !k_cache || !v_cache || !seq_lens || !out) return MQA_ERR_NULL;
    const mqa_status st = check_sizes(b, h, g, S, d, dt, split_chunk);
    if (st != MQA_OK) return st;
    if (workspace_need(b, h, g, S, d, dt, split_chunk, MQA_KERNEL_AUTO) > kScratchBytes)
        return MQA_ERR_SCRATCH;
    void *ws = nullptr;
    if (scratch_of_current_device(&ws) != MQA_OK) return MQA_ERR_HIP;
    return mqa_decode_attn_kernel(q, k_cache, v_cache, seq_lens, b, h, g, S, d, dt, scale, out, ws,
                                  kScratchBytes, split_chunk, err_flags, MQA_KERNEL_AUTO, stream);
}

// ---- several query tokens per sequence ----

size_t mqa_decode_multi_workspace_bytes(int b, int T, int h, int g, int S, int d, mqa_dtype dt,
                                        int split_chunk) {
    if (T == 1) return mqa_decode_workspace_bytes(b, h, g, S, d, dt, split_chunk);
    if (check_sizes(b, h, g, S, d, dt, split_chunk) != MQA_OK) return 0;
    if (check_tokens(T, h, S, dt) != MQA_OK) return 0;
    return workspace_need(b, h, g, S, d, dt, split_chunk, MQA_KERNEL_MFMA, T);
}

int mqa_decode_multi_schedule(int b, int T, int h, int g, int S, int d, mqa_dtype dt,
                              int split_chunk) {
    if (T == 1) return mqa_decode_schedule(b, h, g, S, d, dt, split_chunk, MQA_KERNEL_AUTO);
    if (check_sizes(b, h, g, S, d, dt, split_chunk) != MQA_OK) return -1;
    if (check_tokens(T, h, S, dt) != MQA_OK) return -1;
    return use_streamk(b, h, g, S, dt, split_chunk, MQA_KERNEL_MFMA, T) ? MQA_SCHEDULE_MFMA_BALANCED
                                                                         : MQA_SCHEDULE_MFMA_PARTITIONS;
}

mqa_status mqa_decode_attn_multi(const void *q, const void *k_cache, const void *v_cache,
                                 const int32_t *seq_lens, int b, int T, int h, int g, int S, int d,
                                 mqa_dtype dt, float scale, float *out, void *workspace,
                                 size_t workspace_bytes, int split_chunk, int32_t *err_flags,
                                 hipStream_t stream) {
    if (T == 1)
        return mqa_decode_attn(q, k_cache, v_cache, seq_lens, b, h, g, S, d, dt, scale, out,
                               workspace, workspace_bytes, split_chunk, err_flags, stream);
    if (!q || !k_cache || !v_cache || !seq_lens || !out) return MQA_ERR_NULL;
    mqa_status st = check_sizes(b, h, g, S, d, dt, split_chunk);
    if (st != MQA_OK) return st;
    if ((st = check_tokens(T, h, S, dt)) != MQA_OK) return st;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return MQA_ERR_ALIGN;
    const int chunk = resolve_chunk(b, h, g, S, dt, split_chunk, T);
    const int nsplit = (S + chunk - 1) / chunk;
    if (!workspace || workspace_bytes < workspace_need(b, h, g, S, d, dt, split_chunk, MQA_KERNEL_MFMA, T))
        return MQA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MQA_ERR_ALIGN;
    const bool bal = use_streamk(b, h, g, S, dt, split_chunk, MQA_KERNEL_MFMA, T);
    const float qs = scale * kLog2e;
    const uint8_t *kb = (const uint8_t *)k_cache, *vb = (const uint8_t *)v_cache;
    if (d == 128)
        return run_mfma<128>(ContigKV<128>{kb, vb, g, S}, q, seq_lens, b, T, h, g, S, qs, out,
                             workspace, chunk, nsplit, bal, err_flags, stream);
    return run_mfma<64>(ContigKV<64>{kb, vb, g, S}, q, seq_lens, b, T, h, g, S, qs, out, workspace,
                        chunk, nsplit, bal, err_flags, stream);
}

// ---- paged cache ----

namespace {
mqa_status check_paged(int b, int h, int g, int P, int max_pages, int num_pages, int d,
                       mqa_dtype dt, int split_chunk) {
    if (P < 16 || P % 16 != 0 || max_pages < 1 || num_pages < 1) return MQA_ERR_SHAPE;
    if ((long long)P * max_pages > (1ll << 30)) return MQA_ERR_SHAPE;
    const mqa_status st = check_sizes(b, h, g, P * max_pages, d, dt, split_chunk);
    if (st != MQA_OK) return st;
    if (dt != MQA_BF16) return MQA_ERR_UNSUPPORTED;  // paged reads: matrix-core kernels, bf16
    return MQA_OK;
}
}  // namespace

mqa_status mqa_append_kv_paged_multi(void *k_pages, void *v_pages, const void *k_new,
                                     const void *v_new, const int32_t *block_table,
                                     const int32_t *seq_lens, int b, int T, int g, int page_size,
                                     int max_pages, int num_pages, int d, mqa_dtype dt,
                                     int32_t *err_flags, hipStream_t stream) {
    if (!k_pages || !v_pages || !k_new || !v_new || !block_table || !seq_lens) return MQA_ERR_NULL;
    if (page_size < 1 || max_pages < 1 || num_pages < 1) return MQA_ERR_SHAPE;
    if ((long long)page_size * max_pages > (1ll << 30)) return MQA_ERR_SHAPE;
    const mqa_status st = check_sizes(b, g, g, page_size * max_pages, d, dt, 0);
    if (st != MQA_OK) return st;
    if (T < 1 || T > page_size * max_pages) return MQA_ERR_SHAPE;
    if (!aligned16(k_pages) || !aligned16(v_pages) || !aligned16(k_new) || !aligned16(v_new))
        return MQA_ERR_ALIGN;
    const int row_bytes = d * (dt == MQA_BF16 ? 2 : 4);
    const long long total = 2ll * b * T * g * (row_bytes / 16);
    if ((total + 255) / 256 > 0x7fffffffll) return MQA_ERR_SHAPE;
    MQA_LAUNCH(append_kv_paged_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), stream, (uint8_t *)k_pages, (uint8_t *)v_pages, (const uint8_t *)k_new, (const uint8_t *)v_new, block_table, seq_lens, b, T, g, page_size, max_pages, num_pages, row_bytes, err_flags);
    return MQA_OK;
}

mqa_status mqa_append_kv_paged(void *k_pages, void *v_pages, const void *k_new, const void *v_new,
                               const int32_t *block_table, const int32_t *seq_lens, int b, int g,
                               int page_size, int max_pages, int num_pages, int d, mqa_dtype dt,
                               int32_t *err_flags, hipStream_t stream) {
    return mqa_append_kv_paged_multi(k_pages, v_pages, k_new, v_new, block_table, seq_lens, b, 1,
                                     g, page_size, max_pages, num_pages, d, dt, err_flags, stream);
}

size_t mqa_decode_paged_workspace_bytes(int b, int h, int g, int page_size, int max_pages, int d,
                                        mqa_dtype dt, int split_chunk) {
    if (check_paged(b, h, g, page_size, max_pages, 1, d, dt, split_chunk) != MQA_OK) return 0;
    return workspace_need(b, h, g, page_size * max_pages, d, dt, split_chunk, MQA_KERNEL_MFMA);
}

mqa_status mqa_decode_attn_paged_multi(const void *q, const void *k_pages, const void *v_pages,
                                       const int32_t *block_table, const int32_t *seq_lens, int b,
                                       int T, int h, int g, int page_size, int max_pages,
                                       int num_pages, int d, mqa_dtype dt, float scale, float *out,
                                       void *workspace, size_t workspace_bytes, int split_chunk,
                                       int32_t *err_flags, hipStream_t stream) {
    if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !out) return MQA_ERR_NULL;
    mqa_status st = check_paged(b, h, g, page_size, max_pages, num_pages, d, dt, split_chunk);
    if (st != MQA_OK) return st;
    const int S = page_size * max_pages;
    if ((st = check_tokens(T, h, S, dt)) != MQA_OK) return st;
    if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(out))
        return MQA_ERR_ALIGN;
    const int chunk = resolve_chunk(b, h, g, S, dt, split_chunk, T);
    const int nsplit = (S + chunk - 1) / chunk;
    if (!workspace ||
        workspace_bytes < workspace_need(b, h, g, S, d, dt, split_chunk, MQA_KERNEL_MFMA, T))
        return MQA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MQA_ERR_ALIGN;
    const bool bal = use_streamk(b, h, g, S, dt, split_chunk, MQA_KERNEL_MFMA, T);
    const float qs = scale * kLog2e;
    const uint8_t *kb = (const uint8_t *)k_pages, *vb = (const uint8_t *)v_pages;
    if (d == 128)
        return run_mfma<128>(PagedKV<128>{kb, vb, block_table, g, page_size, max_pages, num_pages}, q,
                             seq_lens, b, T, h, g, S, qs, out, workspace, chunk, nsplit, bal,
                             err_flags, stream);
    return run_mfma<64>(PagedKV<64>{kb, vb, block_table, g, page_size, max_pages, num_pages}, q,
                        seq_lens, b, T, h, g, S, qs, out, workspace, chunk, nsplit, bal, err_flags,
                        stream);
}

mqa_status mqa_decode_attn_paged(const void *q, const void *k_pages, const void *v_pages,
                                 const int32_t *block_table, const int32_t *seq_lens, int b, int h,
                                 int g, int page_size, int max_pages, int num_pages, int d,
                                 mqa_dtype dt, float scale, float *out, void *workspace,
                                 size_t workspace_bytes, int split_chunk, int32_t *err_flags,
                                 hipStream_t stream) {
    return mqa_decode_attn_paged_multi(q, k_pages, v_pages, block_table, seq_lens, b, 1, h, g,
                                       page_size, max_pages, num_pages, d, dt, scale, out,
                                       workspace, workspace_bytes, split_chunk, err_flags, stream);
}

// ---- fp8 e4m3 and int8 caches with per-K/V-head scales ----

extern "C++" {
namespace {
template <bool I8>
mqa_status launch_append_codes(void *k, void *v, const void *k_new, const void *v_new,
                               const float *k_scale, const float *v_scale, const int32_t *bt,
                               const int32_t *seq_lens, int b, int T, int g, int S, int max_pages,
                               int num_pages, int d, int32_t *err_flags, hipStream_t stream) {
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_new) || !aligned16(v_new) ||
        ((uintptr_t)k_scale & 3u) || ((uintptr_t)v_scale & 3u))
        return MQA_ERR_ALIGN;
    const long long total = 2ll * b * T * g * (d / 8);
    if ((total + 255) / 256 > 0x7fffffffll) return MQA_ERR_SHAPE;
    MQA_LAUNCH(append_kv_codes_kernel<I8>, dim3((unsigned)((total + 255) / 256)), dim3(256), stream, (uint8_t *)k, (uint8_t *)v, (const uint16_t *)k_new, (const uint16_t *)v_new, k_scale, v_scale, bt, seq_lens, b, T, g, S, max_pages, num_pages, d, err_flags);
    return MQA_OK;
}

// sizes of an fp8-cache call (q, k_new, v_new are bf16; the cache rows are
// d bytes, checked here as if bf16, which is stricter)
mqa_status check_fp8(int b, int T, int h, int g, int S, int d, int split_chunk) {
    const mqa_status st = check_sizes(b, h, g, S, d, MQA_BF16, split_chunk);
    if (st != MQA_OK) return st;
    return check_tokens(T, h, S, MQA_BF16);
}
}  // namespace
}  // extern "C++"

mqa_status mqa_append_kv_fp8(void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                             const float *k_scale, const float *v_scale, const int32_t *seq_lens,
                             int b, int T, int g, int S, int d, int32_t *err_flags,
                             hipStream_t stream) {
    if (!k_cache || !v_cache || !k_new || !v_new || !k_scale || !v_scale || !seq_lens)
        return MQA_ERR_NULL;
    const mqa_status st = check_fp8(b, T, g, g, S, d, 0);
    if (st != MQA_OK) return st;
    return launch_append_codes<false>(k_cache, v_cache, k_new, v_new, k_scale, v_scale, nullptr,
                                      seq_lens, b, T, g, S, 1, 1, d, err_flags, stream);
}

mqa_status mqa_append_kv_paged_fp8(void *k_pages, void *v_pages, const void *k_new,
                                   const void *v_new, const float *k_scale, const float *v_scale,
                                   const int32_t *block_table, const int32_t *seq_lens, int b,
                                   int T, int g, int page_size, int max_pages, int num_pages,
                                   int d, int32_t *err_flags, hipStream_t stream) {
    if (!k_pages || !v_pages || !k_new || !v_new || !k_scale || !v_scale || !block_table ||
        !seq_lens)
        return MQA_ERR_NULL;
    if (page_size < 1 || max_pages < 1 || num_pages < 1 ||
        (long long)page_size * max_pages > (1ll << 30))
        return MQA_ERR_SHAPE;
    const mqa_status st = check_fp8(b, T, g, g, page_size * max_pages, d, 0);
    if (st != MQA_OK) return st;
    return launch_append_codes<false>(k_pages, v_pages, k_new, v_new, k_scale, v_scale,
                                      block_table, seq_lens, b, T, g, page_size, max_pages,
                                      num_pages, d, err_flags, stream);
}

mqa_status mqa_append_kv_int8(void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                              const float *k_scale, const float *v_scale, const int32_t *seq_lens,
                              int b, int T, int g, int S, int d, int32_t *err_flags,
                              hipStream_t stream) {
    if (!k_cache || !v_cache || !k_new || !v_new || !k_scale || !v_scale || !seq_lens)
        return MQA_ERR_NULL;
    const mqa_status st = check_fp8(b, T, g, g, S, d, 0);
    if (st != MQA_OK) return st;
    return launch_append_codes<true>(k_cache, v_cache, k_new, v_new, k_scale, v_scale, nullptr,
                                     seq_lens, b, T, g, S, 1, 1, d, err_flags, stream);
}

mqa_status mqa_append_kv_paged_int8(void *k_pages, void *v_pages, const void *k_new,
                                    const void *v_new, const float *k_scale, const float *v_scale,
                                    const int32_t *block_table, const int32_t *seq_lens, int b,
                                    int T, int g, int page_size, int max_pages, int num_pages,
                                    int d, int32_t *err_flags, hipStream_t stream) {
    if (!k_pages || !v_pages || !k_new || !v_new || !k_scale || !v_scale || !block_table ||
        !seq_lens)
        return MQA_ERR_NULL;
    if (page_size < 1 || max_pages < 1 || num_pages < 1 ||
        (long long)page_size * max_pages > (1ll << 30))
        return MQA_ERR_SHAPE;
    const mqa_status st = check_fp8(b, T, g, g, page_size * max_pages, d, 0);
    if (st != MQA_OK) return st;
    return launch_append_codes<true>(k_pages, v_pages, k_new, v_new, k_scale, v_scale,
                                     block_table, seq_lens, b, T, g, page_size, max_pages,
                                     num_pages, d, err_flags, stream);
}

mqa_status mqa_decode_attn_fp8(const void *q, const void *k_cache, const void *v_cache,
                               const float *k_scale, const float *v_scale,
                               const int32_t *seq_lens, int b, int T, int h, int g, int S, int d,
                               float scale, float *out, void *workspace, size_t workspace_bytes,
                               int split_chunk, int32_t *err_flags, hipStream_t stream) {
    if (!q || !k_cache || !v_cache || !k_scale || !v_scale || !seq_lens || !out)
        return MQA_ERR_NULL;
    mqa_status st = check_fp8(b, T, h, g, S, d, split_chunk);
    if (st != MQA_OK) return st;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        ((uintptr_t)k_scale & 3u) || ((uintptr_t)v_scale & 3u))
        return MQA_ERR_ALIGN;
    const mqa_dtype dt = MQA_BF16;
    const int chunk = resolve_chunk(b, h, g, S, dt, split_chunk, T);
    const int nsplit = (S + chunk - 1) / chunk;
    if (!workspace || workspace_bytes < workspace_need(b, h, g, S, d, dt, split_chunk, MQA_KERNEL_MFMA, T))
        return MQA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MQA_ERR_ALIGN;
    const bool bal = use_streamk(b, h, g, S, dt, split_chunk, MQA_KERNEL_MFMA, T);
    const float qs = scale * kLog2e;
    const uint8_t *kb = (const uint8_t *)k_cache, *vb = (const uint8_t *)v_cache;
    if (d == 128)
        return run_mfma<128>(ContigKV<128, true>{kb, vb, g, S}, q, seq_lens, b, T, h, g, S, qs, out,
                             workspace, chunk, nsplit, bal, err_flags, stream, k_scale, v_scale);
    return run_mfma<64>(ContigKV<64, true>{kb, vb, g, S}, q, seq_lens, b, T, h, g, S, qs, out,
                        workspace, chunk, nsplit, bal, err_flags, stream, k_scale, v_scale);
}

mqa_status mqa_decode_attn_paged_fp8(const void *q, const void *k_pages, const void *v_pages,
                                     const float *k_scale, const float *v_scale,
                                     const int32_t *block_table, const int32_t *seq_lens, int b,
                                     int T, int h, int g, int page_size, int max_pages,
                                     int num_pages, int d, float scale, float *out, void *workspace,
                                     size_t workspace_bytes, int split_chunk, int32_t *err_flags,
                                     hipStream_t stream) {
    if (!q || !k_pages || !v_pages || !k_scale || !v_scale || !block_table || !seq_lens || !out)
        return MQA_ERR_NULL;
    mqa_status st = check_paged(b, h, g, page_size, max_pages, num_pages, d, MQA_BF16, split_chunk);
    if (st != MQA_OK) return st;
    const int S = page_size * max_pages;
    if ((st = check_tokens(T, h, S, MQA_BF16)) != MQA_OK) return st;
    if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(out) ||
        ((uintptr_t)k_scale & 3u) || ((uintptr_t)v_scale & 3u))
        return MQA_ERR_ALIGN;
    const mqa_dtype dt = MQA_BF16;
    const int chunk = resolve_chunk(b, h, g, S, dt, split_chunk, T);
    const int nsplit = (S + chunk - 1) / chunk;
    if (!workspace || workspace_bytes < workspace_need(b, h, g, S, d, dt, split_chunk, MQA_KERNEL_MFMA, T))
        return MQA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MQA_ERR_ALIGN;
    const bool bal = use_streamk(b, h, g, S, dt, split_chunk, MQA_KERNEL_MFMA, T);
    const float qs = scale * kLog2e;
    const uint8_t *kb = (const uint8_t *)k_pages, *vb = (const uint8_t *)v_pages;
    if (d == 128)
        return run_mfma<128>(PagedKV<128, true>{kb, vb, block_table, g, page_size, max_pages, num_pages},
                             q, seq_lens, b, T, h, g, S, qs, out, workspace, chunk, nsplit, bal,
                             err_flags, stream, k_scale, v_scale);
    return run_mfma<64>(PagedKV<64, true>{kb, vb, block_table, g, page_size, max_pages, num_pages}, q,
                        seq_lens, b, T, h, g, S, qs, out, workspace, chunk, nsplit, bal, err_flags,
                        stream, k_scale, v_scale);
}

// ---- every option at once; rotary position embedding ----

extern "C++" {
namespace {
// Validate a descriptor; on success S is the capacity (paged: P * max_pages).
// sizes_only: the workspace query, which reads the shape fields and the
// presence of block_table but no data pointer
mqa_status check_desc(const mqa_decode_desc *ds, int &S, bool sizes_only = false) {
    if (!ds) return MQA_ERR_NULL;
    if (!sizes_only && (!ds->q || !ds->k || !ds->v || !ds->seq_lens || !ds->out))
        return MQA_ERR_NULL;
    if (ds->window < 0 || ds->T < 1) return MQA_ERR_SHAPE;
    const bool paged = ds->block_table != nullptr;
    const int kd = ds->kv_dtype;
    const bool codes = kd == MQA_FP8_E4M3 || kd == MQA_INT8;  // one-byte codes with scales
    if (kd != MQA_F32 && kd != MQA_BF16 && !codes) return MQA_ERR_UNSUPPORTED;
    if (kd == MQA_F32 && (paged || ds->T != 1 || ds->window != 0)) return MQA_ERR_UNSUPPORTED;
    if (!sizes_only && codes && (!ds->k_scale || !ds->v_scale)) return MQA_ERR_NULL;
    mqa_status st;
    if (paged) {
        st = check_paged(ds->b, ds->h, ds->g, ds->page_size, ds->max_pages, ds->num_pages, ds->d,
                         MQA_BF16, ds->split_chunk);
        S = ds->page_size * ds->max_pages;
    } else {
        st = check_sizes(ds->b, ds->h, ds->g, ds->S, ds->d, kd == MQA_F32 ? MQA_F32 : MQA_BF16,
                         ds->split_chunk);
        S = ds->S;
    }
    if (st != MQA_OK) return st;
    if (kd != MQA_F32 && (st = check_tokens(ds->T, ds->h, S, MQA_BF16)) != MQA_OK) return st;
    if (sizes_only) return MQA_OK;
    if (!aligned16(ds->q) || !aligned16(ds->k) || !aligned16(ds->v) || !aligned16(ds->out))
        return MQA_ERR_ALIGN;
    if (codes && (((uintptr_t)ds->k_scale & 3u) || ((uintptr_t)ds->v_scale & 3u)))
        return MQA_ERR_ALIGN;
    return MQA_OK;
}

template <int D, bool F8, bool I8 = false>
mqa_status run_desc(const mqa_decode_desc *ds, int S, int chunk, int nsplit, bool bal, float qs,
                    hipStream_t stream) {
    const uint8_t *kb = (const uint8_t *)ds->k, *vb = (const uint8_t *)ds->v;
    if (ds->block_table)
        return run_mfma<D>(PagedKV<D, F8, I8>{kb, vb, ds->block_table, ds->g, ds->page_size,
                                              ds->max_pages, ds->num_pages},
                           ds->q, ds->seq_lens, ds->b, ds->T, ds->h, ds->g, S, qs, ds->out,
                           ds->workspace, chunk, nsplit, bal, ds->err_flags, stream, ds->k_scale,
                           ds->v_scale, ds->window);
    return run_mfma<D>(ContigKV<D, F8, I8>{kb, vb, ds->g, S}, ds->q, ds->seq_lens, ds->b, ds->T, ds->h,
                       ds->g, S, qs, ds->out, ds->workspace, chunk, nsplit, bal, ds->err_flags,
                       stream, ds->k_scale, ds->v_scale, ds->window);
}
}  // namespace
}  // extern "C++"

size_t mqa_decode_ex_workspace_bytes(const mqa_decode_desc *ds) {
    int S = 0;
    if (check_desc(ds, S, true) != MQA_OK) return 0;
    if (ds->kv_dtype == MQA_F32)
        return workspace_need(ds->b, ds->h, ds->g, S, ds->d, MQA_F32, ds->split_chunk,
                              MQA_KERNEL_AUTO);
    return workspace_need(ds->b, ds->h, ds->g, window_span(S, ds->T, ds->window), ds->d, MQA_BF16,
                          ds->split_chunk, MQA_KERNEL_MFMA, ds->T);
}

mqa_status mqa_decode_attn_ex(const mqa_decode_desc *ds, hipStream_t stream) {
    int S = 0;
    const mqa_status st = check_desc(ds, S);
    if (st != MQA_OK) return st;
    if (ds->kv_dtype == MQA_F32)
        return mqa_decode_attn(ds->q, ds->k, ds->v, ds->seq_lens, ds->b, ds->h, ds->g, S, ds->d,
                               MQA_F32, ds->scale, ds->out, ds->workspace, ds->workspace_bytes,
                               ds->split_chunk, ds->err_flags, stream);
    const mqa_dtype dt = MQA_BF16;
    const int Sw = window_span(S, ds->T, ds->window);  // what the partitions cover
    const int chunk = resolve_chunk(ds->b, ds->h, ds->g, Sw, dt, ds->split_chunk, ds->T);
    const int nsplit = (Sw + chunk - 1) / chunk;
    if (!ds->workspace || ds->workspace_bytes < workspace_need(ds->b, ds->h, ds->g, Sw, ds->d, dt,
                                                               ds->split_chunk, MQA_KERNEL_MFMA, ds->T))
        return MQA_ERR_WORKSPACE;
    if (!aligned16(ds->workspace)) return MQA_ERR_ALIGN;
    const bool bal = use_streamk(ds->b, ds->h, ds->g, Sw, dt, ds->split_chunk, MQA_KERNEL_MFMA, ds->T);
    const float qs = ds->scale * kLog2e;
    const int kd = ds->kv_dtype;
    if (ds->d == 128)
        return kd == MQA_INT8       ? run_desc<128, true, true>(ds, S, chunk, nsplit, bal, qs, stream)
               : kd == MQA_FP8_E4M3 ? run_desc<128, true>(ds, S, chunk, nsplit, bal, qs, stream)
                                    : run_desc<128, false>(ds, S, chunk, nsplit, bal, qs, stream);
    return kd == MQA_INT8       ? run_desc<64, true, true>(ds, S, chunk, nsplit, bal, qs, stream)
           : kd == MQA_FP8_E4M3 ? run_desc<64, true>(ds, S, chunk, nsplit, bal, qs, stream)
                                : run_desc<64, false>(ds, S, chunk, nsplit, bal, qs, stream);
}

mqa_status mqa_rope_q(void *q, const float *cos_sin, int n_pos, const int32_t *seq_lens, int b,
                      int T, int h, int d, int32_t *err_flags, hipStream_t stream) {
    if (!q || !cos_sin || !seq_lens) return MQA_ERR_NULL;
    if (b < 1 || T < 1 || h < 1 || n_pos < 1) return MQA_ERR_SHAPE;
    if (d != 64 && d != 128) return MQA_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(cos_sin)) return MQA_ERR_ALIGN;
    const long long total = (long long)b * T * h * (d / 16);
    if ((total + 255) / 256 > 0x7fffffffll) return MQA_ERR_SHAPE;
    MQA_LAUNCH(rope_q_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), stream, (uint16_t *)q, cos_sin, n_pos, seq_lens, b, T, h, d, err_flags);
    return MQA_OK;
}

mqa_status mqa_append_kv_rope(void *k_cache, void *v_cache, const void *k_new,
                              const void *v_new, const float *cos_sin, int n_pos,
                              const int32_t *seq_lens, int b, int T, int g, int S, int d,
                              int32_t *err_flags, hipStream_t stream) {
    if (!k_cache || !v_cache || !k_new || !v_new || !cos_sin || !seq_lens) return MQA_ERR_NULL;
    mqa_status st = check_sizes(b, g, g, S, d, MQA_BF16, 0);
    if (st != MQA_OK) return st;
    if (T < 1 || T > S || n_pos < 1) return MQA_ERR_SHAPE;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new) ||
        !aligned16(cos_sin))
        return MQA_ERR_ALIGN;
    const long long total = (long long)b * T * g * (d / 16);
    if ((total + 255) / 256 > 0x7fffffffll) return MQA_ERR_SHAPE;
    MQA_LAUNCH(append_kv_rope_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), stream, (uint16_t *)k_cache, (uint16_t *)v_cache, (const uint16_t *)k_new, (const uint16_t *)v_new, cos_sin, n_pos, seq_lens, b, T, g, S, d, err_flags);
    return MQA_OK;
}

}  // extern "C"

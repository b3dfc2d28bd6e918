// libmqa_decode: decode attention over a shared-head KV cache on gfx950.
//
// One decode step ([GQA notes] = ybb.press "分组查询注意力（GQA）与多查询注意力
// （MQA）深度实战"): append the new token's K/V to the cache (§八; nanhubrain.csdn.net
// MQA article §2.2), then for every query head hq of every sequence i, with
// G = h/g query heads per K/V head and j = hq / G (§五),
//   out[i,hq,:] = softmax_t(scale * q[i,hq,:] . K[i,j,t,:]) V[i,j,t,:],  t < L_i.
//
// Kernels
//   append_kv_kernel     one 16-byte chunk per thread, bit copy.
//   split_rows_kernel    one work-group per (partition of the sequence, K/V head,
//                        block of up to 8 query heads, sequence). The K and V
//                        tiles of 64 cache rows are copied global->LDS with
//                        128-bit DMA loads, read from HBM once, and reused by
//                        every query head of the group. Scores: one wave per
//                        query head, one lane per cache row, bf16 dot2 FMAs.
//                        Online softmax (running max / sum) per head; P.V with
//                        fp32 FMAs, each lane owning one 16-byte column chunk.
//                        Writes the partition's (max, sum, unnormalised o).
//   combine_kernel       log-sum-exp merge of the partitions into out.
//
// Everything is enqueued on the caller's stream; nothing is allocated here.

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Wait until at most N vector-memory operations of this wave are pending,
// then work-group barrier.
template <int N>
__device__ __forceinline__ void vmem_wait_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(N) : "memory");
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

// Thread t copies one 16-byte chunk: t -> (tensor K/V, sequence i, head j, chunk c).
__global__ void append_kv_kernel(uint8_t *__restrict__ kc, uint8_t *__restrict__ vc,
                                 const uint8_t *__restrict__ kn, const uint8_t *__restrict__ vn,
                                 const int32_t *__restrict__ seq_lens, int b, int g, int S,
                                 int row_bytes, int32_t *__restrict__ err) {
    const int cpr = row_bytes >> 4;
    const long long total = 2ll * b * g * cpr;
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= total) return;
    const int c = (int)(t % cpr);
    const long long ij = (t / cpr) % ((long long)b * g);
    const int which = (int)(t / ((long long)cpr * b * g));
    const int i = (int)(ij / g);
    const int L = seq_lens[i];
    if (L < 1 || L > S) {
        if (c == 0 && which == 0 && (ij % g) == 0 && err) atomicOr(err, MQA_DEVERR_SEQLEN);
        return;
    }
    const size_t src = (size_t)ij * row_bytes + (size_t)c * 16;
    const size_t dst = ((size_t)ij * S + (size_t)(L - 1)) * row_bytes + (size_t)c * 16;
    const uint8_t *s = which ? vn : kn;
    uint8_t *dp = which ? vc : kc;
    *(uint4 *)(dp + dst) = *(const uint4 *)(s + src);
}

// ---------------------------------------------------------------------------
// split kernel: one wave per query head in the score phase, one lane per row
// ---------------------------------------------------------------------------

template <typename T, int D, int HPW>
struct RowsCfg {
    static constexpr int EB = (int)sizeof(T);
    static constexpr int ROW_BYTES = D * EB;          // 128 .. 512
    static constexpr int CPR = ROW_BYTES / 16;        // 16-byte chunks per row
    static constexpr int ELEMS = 16 / EB;             // elements per chunk
    static constexpr int NW = HPW;                    // waves per work-group
    static constexpr int NT = 64 * NW;
    static constexpr int TILE_BYTES = kTile * ROW_BYTES;
    static constexpr int DMA = TILE_BYTES / 16 / NT;  // DMA loads per lane per K (or V) tile
    static constexpr int RPW = kTile / NW;            // rows per wave in the P.V phase
    static constexpr int RPI = 64 / CPR;              // rows covered by one wave-wide 1 KB
    static constexpr int VROWS = RPW / RPI;           // rows per lane in the P.V phase
    static constexpr int ROW_DW = ROW_BYTES / 4;
    static_assert(DMA >= 1 && VROWS >= 1, "too many waves for this row size");
    static_assert(NW * HPW * D * 4 <= 2 * 2 * TILE_BYTES, "reduction scratch must fit");
};

template <typename T, int D, int HPW>
struct RowsSmem {
    using C = RowsCfg<T, D, HPW>;
    uint8_t kv[2][2][C::TILE_BYTES];  // [stage][K=0, V=1], rows XOR-swizzled in 16-byte chunks
    float p[kTile][HPW];              // softmax numerators of the current tile, [row][head]
    float alpha[HPW];                 // rescale factor of the running sums, per head
};

// Issue the DMA of one 64-row tile of K or V into LDS. Row r, chunk c lands at
// r*ROW_BYTES + 16*(c ^ (r % CPR)): a 64-lane read of one chunk of 64 rows, or
// of 64 chunks of 4 rows, touches 64 distinct 16-byte bank groups.
template <typename C>
__device__ __forceinline__ void dma_tile(const uint8_t *__restrict__ base, int t0, int S,
                                         uint8_t *lds_tile, int w, int lane) {
#pragma unroll
    for (int r = 0; r < C::DMA; r++) {
        const int blk = w * C::DMA + r;  // 1 KB block of the tile written by this instruction
        const int slot = blk * 64 + lane;
        const int row = slot / C::CPR;
        const int chunk = (slot % C::CPR) ^ (row % C::CPR);
        const int grow = min(t0 + row, S - 1);  // rows past the capacity are never used
        dma16(base + (size_t)grow * C::ROW_BYTES + chunk * 16, lds_addr(lds_tile + blk * 1024));
    }
}

template <typename T, int D, int HPW>
__global__ void __launch_bounds__(64 * HPW)
split_rows_kernel(const T *__restrict__ q, const T *__restrict__ kc, const T *__restrict__ vc,
                  const int32_t *__restrict__ seq_lens, int h, int g, int S, int G, int nhc,
                  int chunk, int nsplit, float qk_scale_log2, float *__restrict__ part_o,
                  float2 *__restrict__ part_ml) {
    using C = RowsCfg<T, D, HPW>;
    __shared__ __attribute__((aligned(16))) RowsSmem<T, D, HPW> sm;

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
    // are never written out).
    const int slot_w = hc * HPW + w;
    const int hq_w = j * G + min(slot_w, G - 1);
    const uint32_t *qrow = (const uint32_t *)(q + ((size_t)i * h + hq_w) * D);
    uint32_t qv[C::ROW_DW];
#pragma unroll
    for (int x = 0; x < C::ROW_DW; x++) qv[x] = qrow[x];

    // P.V ownership: lane -> (row group rg, 16-byte column chunk cc)
    const int rg = lane / C::CPR;
    const int cc = lane % C::CPR;

    float acc[HPW][C::ELEMS];
#pragma unroll
    for (int a = 0; a < HPW; a++)
#pragma unroll
        for (int e = 0; e < C::ELEMS; e++) acc[a][e] = 0.f;
    float m_run = -INFINITY;  // running max of this wave's head (log2 units)
    float l_lane = 0.f;       // this lane's share of the running sum

    dma_tile<C>(kbase, t_begin, S, sm.kv[0][0], w, lane);
    dma_tile<C>(vbase, t_begin, S, sm.kv[0][1], w, lane);

    for (int n = 0; n < ntiles; n++) {
        const int st = n & 1;
        const int t0 = t_begin + n * kTile;
        // tile n landed everywhere; every wave finished tile n-1
        vmem_wait_barrier<0>();
        if (n + 1 < ntiles) {
            dma_tile<C>(kbase, t0 + kTile, S, sm.kv[st ^ 1][0], w, lane);
            dma_tile<C>(vbase, t0 + kTile, S, sm.kv[st ^ 1][1], w, lane);
        }

        // ---- scores: lane = cache row, wave = query head ----
        const uint8_t *krow = sm.kv[st][0] + lane * C::ROW_BYTES;
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
        for (int c = 0; c < C::CPR; c++) {
            const uint4 kk = *(const uint4 *)(krow + ((c ^ (lane % C::CPR)) << 4));
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
        const bool row_ok = t0 + lane < t_end;
        const float s2 = row_ok ? ((a0 + a1) + (a2 + a3)) * qk_scale_log2 : -INFINITY;
        const float m_new = fmaxf(m_run, wave_max(s2));  // finite: row t0 is always valid
        const float alpha = fast_exp2(m_run - m_new);
        const float p = fast_exp2(s2 - m_new);
        l_lane = l_lane * alpha + p;
        m_run = m_new;
        sm.p[lane][w] = p;
        if (lane == 0) sm.alpha[w] = alpha;
        lds_barrier();

        // ---- P.V: lane owns column chunk cc of rows rg, rg+RPI, ... ----
        float al[HPW];
#pragma unroll
        for (int a = 0; a < HPW; a++) al[a] = sm.alpha[a];
#pragma unroll
        for (int a = 0; a < HPW; a++)
#pragma unroll
            for (int e = 0; e < C::ELEMS; e++) acc[a][e] *= al[a];
#pragma unroll
        for (int r = 0; r < C::VROWS; r++) {
            const int row = w * C::RPW + r * C::RPI + rg;
            const uint4 vv =
                *(const uint4 *)(sm.kv[st][1] + row * C::ROW_BYTES + ((cc ^ (row % C::CPR)) << 4));
            float vf[C::ELEMS];
            if constexpr (sizeof(T) == 2) {
                vf[0] = bf16_lo(vv.x); vf[1] = bf16_hi(vv.x);
                vf[2] = bf16_lo(vv.y); vf[3] = bf16_hi(vv.y);
                vf[4] = bf16_lo(vv.z); vf[5] = bf16_hi(vv.z);
                vf[6] = bf16_lo(vv.w); vf[7] = bf16_hi(vv.w);
            } else {
                vf[0] = __uint_as_float(vv.x); vf[1] = __uint_as_float(vv.y);
                vf[2] = __uint_as_float(vv.z); vf[3] = __uint_as_float(vv.w);
            }
            // rows past the end may hold anything (even NaN): never let them in
            const bool ok = t0 + row < t_end;
#pragma unroll
            for (int e = 0; e < C::ELEMS; e++) vf[e] = ok ? vf[e] : 0.f;
            float pr[HPW];
#pragma unroll
            for (int a = 0; a < HPW; a++) pr[a] = sm.p[row][a];
#pragma unroll
            for (int a = 0; a < HPW; a++)
#pragma unroll
                for (int e = 0; e < C::ELEMS; e++) acc[a][e] = fmaf(pr[a], vf[e], acc[a][e]);
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
            for (int off = C::CPR; off < 64; off <<= 1) x += __shfl_xor(x, off);
            acc[a][e] = x;
        }
    lds_barrier();  // every wave is done with the tiles; reuse them as scratch
    float *red = (float *)&sm.kv[0][0][0];  // [NW][HPW][D]
    if (lane < C::CPR) {
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
        part_ml[hq * nsplit + s] = make_float2(m_run, l_tot);
    }
}

// ---------------------------------------------------------------------------
// combine: out = sum_s 2^(m_s-M) o_s / sum_s 2^(m_s-M) l_s over live partitions
// ---------------------------------------------------------------------------

template <int D>
__global__ void __launch_bounds__(D)
combine_kernel(const float *__restrict__ part_o, const float2 *__restrict__ part_ml,
               const int32_t *__restrict__ seq_lens, int h, int S, int chunk, int nsplit,
               float *__restrict__ out, int32_t *__restrict__ err) {
    const int hq = blockIdx.x, i = blockIdx.y, x = threadIdx.x;
    const size_t row = (size_t)i * h + hq;
    const int L = seq_lens[i];
    if (L < 1 || L > S) {
        out[row * D + x] = __builtin_nanf("");
        if (hq == 0 && x == 0 && err) atomicOr(err, MQA_DEVERR_SEQLEN);
        return;
    }
    const int n = (L + chunk - 1) / chunk;
    const float2 *ml = part_ml + row * nsplit;
    float M = -INFINITY;
    for (int s = 0; s < n; s++) M = fmaxf(M, ml[s].x);
    float num = 0.f, den = 0.f;
    for (int s = 0; s < n; s++) {
        const float2 e = ml[s];
        const float wgt = fast_exp2(e.x - M);
        den = fmaf(wgt, e.y, den);
        num = fmaf(wgt, part_o[(row * nsplit + s) * D + x], num);
    }
    out[row * D + x] = num / den;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTargetGroups = 2048;  // aim for ~8 partitions per compute unit

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
    return MQA_OK;
}

int resolve_chunk(int b, int h, int g, int S, int split_chunk) {
    if (split_chunk > 0) return split_chunk;
    const int G = h / g;
    const long long groups = (long long)b * g * ((G + heads_per_wg(G) - 1) / heads_per_wg(G));
    const long long want = (kTargetGroups + groups - 1) / groups;  // partitions per group
    long long c = ((long long)S + want - 1) / want;
    c = (c + kTile - 1) / kTile * kTile;
    if (c < 256) c = 256;
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

template <typename T, int D, int HPW>
void launch_rows(const void *q, const void *k, const void *v, const int32_t *seq_lens, int b,
                 int h, int g, int S, float qk_scale_log2, int chunk, int nsplit, float *part_o,
                 float2 *part_ml, hipStream_t stream) {
    const int G = h / g;
    const int nhc = (G + HPW - 1) / HPW;
    dim3 grid(nsplit, g * nhc, b);
    hipLaunchKernelGGL((split_rows_kernel<T, D, HPW>), grid, dim3(64 * HPW), 0, stream,
                       (const T *)q, (const T *)k, (const T *)v, seq_lens, h, g, S, G, nhc, chunk,
                       nsplit, qk_scale_log2, part_o, part_ml);
}

template <typename T, int D>
void dispatch_rows(int hpw, const void *q, const void *k, const void *v, const int32_t *seq_lens,
                   int b, int h, int g, int S, float qs, int chunk, int nsplit, float *po,
                   float2 *pml, hipStream_t st) {
    switch (hpw) {
        case 1: launch_rows<T, D, 1>(q, k, v, seq_lens, b, h, g, S, qs, chunk, nsplit, po, pml, st); break;
        case 2: launch_rows<T, D, 2>(q, k, v, seq_lens, b, h, g, S, qs, chunk, nsplit, po, pml, st); break;
        case 4: launch_rows<T, D, 4>(q, k, v, seq_lens, b, h, g, S, qs, chunk, nsplit, po, pml, st); break;
        default: launch_rows<T, D, 8>(q, k, v, seq_lens, b, h, g, S, qs, chunk, nsplit, po, pml, st); break;
    }
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
    }
    return "unknown status";
}

uint64_t mqa_kv_bytes(int layers, int g, int64_t S, int d, int dtype_bytes) {
    if (layers < 0 || g < 0 || S < 0 || d < 0 || dtype_bytes < 0) return 0;
    return 2ull * (uint64_t)layers * (uint64_t)g * (uint64_t)S * (uint64_t)d * (uint64_t)dtype_bytes;
}

int mqa_decode_resolve_chunk(int b, int h, int g, int S, int d, mqa_dtype dt, int split_chunk) {
    if (check_sizes(b, h, g, S, d, dt, split_chunk) != MQA_OK) return -1;
    return resolve_chunk(b, h, g, S, split_chunk);
}

size_t mqa_decode_workspace_bytes(int b, int h, int g, int S, int d, mqa_dtype dt,
                                  int split_chunk) {
    if (check_sizes(b, h, g, S, d, dt, split_chunk) != MQA_OK) return 0;
    return workspace_for(b, h, S, d, resolve_chunk(b, h, g, S, split_chunk));
}

mqa_status mqa_append_kv(void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                         const int32_t *seq_lens, int b, int g, int S, int d, mqa_dtype dt,
                         int32_t *err_flags, hipStream_t stream) {
    if (!k_cache || !v_cache || !k_new || !v_new || !seq_lens) return MQA_ERR_NULL;
    mqa_status st = check_sizes(b, g, g, S, d, dt, 0);
    if (st != MQA_OK) return st;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
        return MQA_ERR_ALIGN;
    const int row_bytes = d * (dt == MQA_BF16 ? 2 : 4);
    const long long total = 2ll * b * g * (row_bytes / 16);
    const int threads = 256;
    const long long blocks = (total + threads - 1) / threads;
    hipLaunchKernelGGL(append_kv_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       (uint8_t *)k_cache, (uint8_t *)v_cache, (const uint8_t *)k_new,
                       (const uint8_t *)v_new, seq_lens, b, g, S, row_bytes, err_flags);
    return hipGetLastError() == hipSuccess ? MQA_OK : MQA_ERR_HIP;
}

mqa_status mqa_decode_attn(const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *seq_lens, int b, int h, int g, int S, int d,
                           mqa_dtype dt, float scale, float *out, void *workspace,
                           size_t workspace_bytes, int split_chunk, int32_t *err_flags,
                           hipStream_t stream) {
    if (!q || !k_cache || !v_cache || !seq_lens || !out) return MQA_ERR_NULL;
    mqa_status st = check_sizes(b, h, g, S, d, dt, split_chunk);
    if (st != MQA_OK) return st;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return MQA_ERR_ALIGN;
    const int chunk = resolve_chunk(b, h, g, S, split_chunk);
    const int nsplit = (S + chunk - 1) / chunk;
    const size_t need = workspace_for(b, h, S, d, chunk);
    if (!workspace || workspace_bytes < need) return MQA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MQA_ERR_ALIGN;

    const size_t rows = (size_t)b * h * nsplit;
    float *part_o = (float *)workspace;
    float2 *part_ml =
        (float2 *)((uint8_t *)workspace + ((rows * d * sizeof(float) + 255) & ~(size_t)255));
    const float qs = scale * kLog2e;
    const int hpw = heads_per_wg(h / g);

    if (dt == MQA_BF16) {
        if (d == 128) dispatch_rows<uint16_t, 128>(hpw, q, k_cache, v_cache, seq_lens, b, h, g, S, qs, chunk, nsplit, part_o, part_ml, stream);
        else dispatch_rows<uint16_t, 64>(hpw, q, k_cache, v_cache, seq_lens, b, h, g, S, qs, chunk, nsplit, part_o, part_ml, stream);
    } else {
        // fp32 rows of 128 elements need at least two waves per work-group
        if (d == 128) dispatch_rows<float, 128>(hpw < 2 ? 2 : hpw, q, k_cache, v_cache, seq_lens, b, h, g, S, qs, chunk, nsplit, part_o, part_ml, stream);
        else dispatch_rows<float, 64>(hpw, q, k_cache, v_cache, seq_lens, b, h, g, S, qs, chunk, nsplit, part_o, part_ml, stream);
    }
    if (hipGetLastError() != hipSuccess) return MQA_ERR_HIP;
    if (d == 128)
        hipLaunchKernelGGL(combine_kernel<128>, dim3(h, b), dim3(128), 0, stream, part_o, part_ml,
                           seq_lens, h, S, chunk, nsplit, out, err_flags);
    else
        hipLaunchKernelGGL(combine_kernel<64>, dim3(h, b), dim3(64), 0, stream, part_o, part_ml,
                           seq_lens, h, S, chunk, nsplit, out, err_flags);
    return hipGetLastError() == hipSuccess ? MQA_OK : MQA_ERR_HIP;
}

}  // extern "C"

// Paged decode attention for gfx950: one query token, GQA, 16-token pages.
//
// The pages describe decode attention as softmax over q.K plus weighted-V
// accumulation, streamed over the KV cache page by page ("The Architecture of
// Modern Inference…", section "Three Critical Engineering Challenges", item 1;
// page size and the 4 KiB kv-head slice in "Building a Custom LLM Inference
// Runtime…", section "Technical Specifications and Hardware Alignment").
// Their Hopper design (one TMA producer warp, six consumer warps, mbarriers)
// is not used: here a work-group owns one kv head and a contiguous range of
// logical pages (split-KV), and each of its waves a quarter of that range,
// for all query heads of the kv head, so every K/V page is read once.  A wave
// requests the K and V of up to 4 pages at once (the page numbers by scalar
// loads first); both products run on the matrix cores.  The waves are merged
// through LDS, the work-group publishes its partial, and the last
// work-group of the kv head merges all splits and writes fp16 outputs.  Every
// barrier is reached by all waves (no barrier in lane- or wave-dependent
// control flow).  Partials are written with device-scope (sc1) stores; every
// wave waits for its stores to be acknowledged before the barrier that
// precedes the arrival atomic, so the last work-group never reads a partial
// before it is complete.
#pragma once

#include "w4_device.hpp"

namespace w4 {

struct AttnProblem {
    const uint16_t *q;          // fp16 [n_qh][128]
    const uint16_t *kpool;      // fp16 [phys][n_kvh][16][128]
    const uint16_t *vpool;
    const int *page_table;
    const int *pos_ptr;         // if set, ctx = *pos_ptr + 1
    int ctx;                    // used when pos_ptr is null
    int n_kvh;
    int pages_per_split;
    int n_split;
    float scale_log2;           // softmax scale * log2(e)
    float *part_ml;             // [n_kvh][n_split][G][2] (max, sum) base-2 domain
    float *part_acc;            // [n_kvh][n_split][G][128]
    unsigned *counter;          // [n_kvh][kAttnCtrStride]: one 128-byte line per kv head
    uint16_t *out;              // fp16 [n_qh][128]
};

// Splits per kv head: about kAttnTargetSplits, each a multiple of the
// work-group's 4 waves in pages and at least kAttnMinPps pages (a short split
// saves page-loop time but adds partials for the last-arriver merge to read).
// Measured per call at context 8192 (512 pages): about 32 splits 14.6 us,
// 64 splits 16.0.
#ifndef W4_ATTN_TARGET_SPLITS
#define W4_ATTN_TARGET_SPLITS 32
#endif
#ifndef W4_ATTN_MIN_PPS
#define W4_ATTN_MIN_PPS 4
#endif
#ifndef W4_ATTN_WAVES
#define W4_ATTN_WAVES 4
#endif
constexpr int kAttnWaves = W4_ATTN_WAVES;      // waves per work-group
constexpr int kAttnThreads = kAttnWaves * 64;
constexpr int kAttnTargetSplits = W4_ATTN_TARGET_SPLITS;
constexpr int kAttnMinPps = W4_ATTN_MIN_PPS;
static_assert(kAttnTargetSplits >= 1 && kAttnTargetSplits <= 256 && kAttnMinPps >= 1, "attention split bounds");
inline int attn_pages_per_split(int n_pages_max) {
    int pps = (n_pages_max + kAttnTargetSplits - 1) / kAttnTargetSplits;
    if (pps < kAttnMinPps) pps = kAttnMinPps;
    return (pps + kAttnWaves - 1) / kAttnWaves * kAttnWaves;
}
inline int attn_n_split(int n_pages_max) {
    const int pps = attn_pages_per_split(n_pages_max);
    return (n_pages_max + pps - 1) / pps;
}

constexpr int kAttnBatch = 4;       // pages whose K and V a wave holds in registers at once
#ifndef W4_ATTN_MERGE_ROUND
#define W4_ATTN_MERGE_ROUND 4
#endif
constexpr int kAttnMergeRound = W4_ATTN_MERGE_ROUND;   // splits per load round of the last-arriver merge
constexpr int kAttnRow = kHeadDim + 8;   // LDS row of the V copy, in halves (padded: no bank conflicts)
constexpr int kAttnSlot = kPage * kAttnRow * 2;   // bytes per wave: V copy, then its merge record
static_assert(kAttnSlot >= 8 * 130 * 4, "a wave's slot holds the merge record of 8 query heads");
static_assert(kAttnWaves * kAttnSlot >= 256 * 8 * 8, "the slots hold the (max, sum) pairs of 256 splits of 8 heads");

// Arrival counters one 128-byte line apart: atomics on one line serialise
// (about 18 ns each), so with the kv heads' counters on one line the 4 x 64
// arrivals of a long context queued behind each other.
constexpr int kAttnCtrStride = 32;

typedef _Float16 attn_h4 __attribute__((ext_vector_type(4)));
typedef float attn_f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ attn_h4 attn_pair(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(attn_h4, static_cast<uint64_t>(a) | (static_cast<uint64_t>(b) << 32));
}
__device__ __forceinline__ float attn_lane(float v, int src) {   // v of lane src
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, v)));
}

// K and V of logical pages [c0, min(c0 + kAttnBatch, pe)) of kv head j: lane
// l holds token l % 16 and dims 32 (l / 16) .. + 31 of each (64 contiguous
// bytes per operand and page).  The page numbers are read with scalar loads,
// all before the K/V loads that need them.
__device__ __forceinline__ void attn_load_batch(const AttnProblem &a, int j, int c0, int pe, int tok, int g4,
                                                u32x4 (&k)[kAttnBatch][4], u32x4 (&v)[kAttnBatch][4]) {
    const size_t slice = static_cast<size_t>(kPage) * kHeadDim;
    const const_u32_ptr pt = as_const(reinterpret_cast<const uint32_t *>(a.page_table));
    int phy[kAttnBatch];
#pragma unroll
    for (int pg = 0; pg < kAttnBatch; ++pg)
        phy[pg] = c0 + pg < pe ? static_cast<int>(pt[__builtin_amdgcn_readfirstlane(c0 + pg)]) : 0;
#pragma unroll
    for (int pg = 0; pg < kAttnBatch; ++pg) {
        if (c0 + pg < pe) {
            const size_t base = (static_cast<size_t>(phy[pg]) * a.n_kvh + j) * slice + tok * kHeadDim + g4 * 32;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                k[pg][q] = *reinterpret_cast<const u32x4 *>(a.kpool + base + q * 8);
                v[pg][q] = *reinterpret_cast<const u32x4 *>(a.vpool + base + q * 8);
            }
        }
    }
}

// One work-group per (kv head j, split sp); its wave w takes the split's
// pages [sp pps + w pps / 4, + pps / 4) for all G query heads of the kv head,
// so each K/V page is read once.  Both products run on the matrix cores
// (v_mfma_f32_16x16x16_f16; lane l holds row l % 16 and k 4 (l / 16) + i of
// A, column l % 16 and the same k of B, rows 4 (l / 16) + i of column l % 16
// of the result):
//  - scores, tokens x heads: A = the page's K (lane: token l % 16, its 32
//    dims loaded as 64 contiguous bytes, 4 of them per step), B = q^T (heads
//    past G are zero).  Both operands run over the dims in the order
//    (step s, lane group g, i) -> dim 32 g + 4 s + i;
//  - P.V, heads x dims: A = the softmax weights, which the score layout
//    already holds as (head l % 16, tokens 4 (l / 16) + i), taken as an fp16
//    pair hi + lo (two products; their sum carries the fp32 weight to about
//    22 bits); B = 16 dims of V, read down the columns of the wave's LDS copy
//    of the page (written row by row).
// Scores are taken in the base-2 exponent domain.  A wave keeps a softmax
// state per head (max, sum, 128 weighted-V sums) over its pages; the waves are
// merged through LDS in wave order, the work-group publishes its partial, and
// the last work-group of the kv head merges all splits in split order.
template <int G>
__global__ __launch_bounds__(kAttnThreads) void attn_decode_kernel(AttnProblem a) {
    static_assert(G >= 1 && G <= 8, "query heads per kv head");
    __shared__ __attribute__((aligned(16))) unsigned char s_slot[kAttnWaves][kAttnSlot];
    __shared__ int s_last;

    const int t = threadIdx.x;
    const int lane = t & 63, wave = wave_id();
    const int r16 = lane & 15, g4 = lane >> 4;
    const int j = blockIdx.x / a.n_split;
    const int sp = blockIdx.x - j * a.n_split;
    const int ctx = a.pos_ptr ? *as_const(reinterpret_cast<const uint32_t *>(a.pos_ptr)) + 1 : a.ctx;
    const int n_pages = (ctx + kPage - 1) / kPage;
    const int ppw = a.pages_per_split / kAttnWaves;
    const int pb = sp * a.pages_per_split + wave * ppw;
    const int pe = min(pb + ppw, n_pages);

    // the first batch of K/V loads goes out before anything else
    u32x4 kr[kAttnBatch][4], vr[kAttnBatch][4];
    if (pb < pe) attn_load_batch(a, j, pb, pe, r16, g4, kr, vr);

    // q^T operand: head r16 (zero past G), dims 32 g4 + 4 s .. + 3 for step s
    uint32_t qb[8][2];
    {
        u32x4 q4[4] = {};
        if (r16 < G) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                q4[q] = *reinterpret_cast<const u32x4 *>(a.q + (j * G + r16) * kHeadDim + g4 * 32 + q * 8);
        }
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const u32x4 w = q4[s >> 1];
            qb[s][0] = (s & 1) ? w.z : w.x;
            qb[s][1] = (s & 1) ? w.w : w.y;
        }
    }

    uint16_t *vcopy = reinterpret_cast<uint16_t *>(s_slot[wave]);
    float m = -INFINITY, lsum = 0.f;        // head r16 (the same in every lane group)
    attn_f4 o[8];                           // heads 4 g4 + i, dims 16 b + r16
#pragma unroll
    for (int b = 0; b < 8; ++b) o[b] = attn_f4{0.f, 0.f, 0.f, 0.f};

    // every batch holds a valid token: its first page is below n_pages
    for (int c0 = pb; c0 < pe; c0 += kAttnBatch) {
        if (c0 != pb) attn_load_batch(a, j, c0, pe, r16, g4, kr, vr);
        attn_f4 sc[kAttnBatch];
        float mb = -INFINITY;
#pragma unroll
        for (int pg = 0; pg < kAttnBatch; ++pg) {
            attn_f4 s4 = {0.f, 0.f, 0.f, 0.f};
            if (c0 + pg < pe) {
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const u32x4 w = kr[pg][s >> 1];
                    const attn_h4 ka = (s & 1) ? attn_pair(w.z, w.w) : attn_pair(w.x, w.y);
                    s4 = __builtin_amdgcn_mfma_f32_16x16x16f16(ka, attn_pair(qb[s][0], qb[s][1]), s4, 0, 0, 0);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = (c0 + pg) * kPage + 4 * g4 + i;
                sc[pg][i] = c0 + pg < pe && tok < ctx ? s4[i] * a.scale_log2 : -INFINITY;
                mb = fmaxf(mb, sc[pg][i]);
            }
        }
        mb = fmaxf(mb, attn_lane(mb, lane ^ 16));
        mb = fmaxf(mb, attn_lane(mb, lane ^ 32));
        const float mn = fmaxf(m, mb);
        const float corr = exp2f(m - mn);   // 0 on the first batch (m = -inf)
        lsum *= corr;
        if (c0 != pb) {
            // rows of o are heads 4 g4 + i: their factors sit in lanes 4 g4 + i
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float f = attn_lane(corr, 4 * g4 + i);
#pragma unroll
                for (int b = 0; b < 8; ++b) o[b][i] *= f;
            }
        }
        m = mn;
#pragma unroll
        for (int pg = 0; pg < kAttnBatch; ++pg) {
            if (c0 + pg >= pe) break;       // uniform over the wave
            attn_h4 ph, pl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pw = exp2f(sc[pg][i] - mn);
                lsum += pw;
                ph[i] = static_cast<_Float16>(pw);
                pl[i] = static_cast<_Float16>(pw - static_cast<float>(ph[i]));
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<u32x4 *>(vcopy + r16 * kAttnRow + g4 * 32 + q * 8) = vr[pg][q];
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                attn_h4 vb;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    vb[i] = __builtin_bit_cast(_Float16, vcopy[(4 * g4 + i) * kAttnRow + 16 * b + r16]);
                o[b] = __builtin_amdgcn_mfma_f32_16x16x16f16(ph, vb, o[b], 0, 0, 0);
                o[b] = __builtin_amdgcn_mfma_f32_16x16x16f16(pl, vb, o[b], 0, 0, 0);
            }
        }
    }
    lsum += attn_lane(lsum, lane ^ 16);
    lsum += attn_lane(lsum, lane ^ 32);

    // this wave's record in its slot: [head][max, sum, 128 sums] for heads < G
    float *rec = reinterpret_cast<float *>(s_slot[wave]);
    if (g4 == 0 && r16 < G) { rec[r16 * 130] = m; rec[r16 * 130 + 1] = lsum; }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = 4 * g4 + i;
        if (h < G) {
#pragma unroll
            for (int b = 0; b < 8; ++b) rec[h * 130 + 2 + 16 * b + r16] = o[b][i];
        }
    }
    __syncthreads();
    // merge the waves in wave order; thread -> (head, dims 2 d2, 2 d2 + 1)
    const size_t pbase = (static_cast<size_t>(j) * a.n_split + sp) * G;
    for (int idx = t; idx < G * 64; idx += kAttnThreads) {
        const int h = idx >> 6, d2 = idx & 63;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, reinterpret_cast<const float *>(s_slot[w])[h * 130]);
        float L = 0.f, A0 = 0.f, A1 = 0.f;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) {
            const float *rw = reinterpret_cast<const float *>(s_slot[w]) + h * 130;
            if (rw[0] != -INFINITY) {
                const float f = exp2f(rw[0] - M);
                L += rw[1] * f;
                A0 += rw[2 + 2 * d2] * f;
                A1 += rw[3 + 2 * d2] * f;
            }
        }
        store_agent(a.part_acc + (pbase + h) * 128 + 2 * d2, A0);
        store_agent(a.part_acc + (pbase + h) * 128 + 2 * d2 + 1, A1);
        if (d2 == 0) {
            store_agent(a.part_ml + (pbase + h) * 2, M);
            store_agent(a.part_ml + (pbase + h) * 2 + 1, L);
        }
    }
    // every wave waits until its partial stores are acknowledged before the
    // barrier, so wave 0's arrival below is ordered after all of them
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t < 64) {
        const bool last = arrive_last(a.counter + j * kAttnCtrStride, static_cast<unsigned>(a.n_split));
        if (t == 0) s_last = last ? 1 : 0;
    }
    __syncthreads();
    if (!s_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

    // merge all splits of kv head j in split order (deterministic).  The
    // partials are complete (their stores were acknowledged before the
    // arrivals) and nothing on this device read them earlier in this launch,
    // so no L2 holds a stale copy and plain 16-byte loads see them.  Lane
    // (h, 4 dims) streams its float4 partials in rounds of kAttnMergeRound
    // splits, the next round's loads in flight while one is summed; the first
    // round goes out together with the (max, sum) pairs (which go through
    // LDS, reusing the slots: they hold n_split * G <= 2176 pairs).  Indices
    // past the last split are clamped (their loads repeat it) and weighted 0,
    // so the loads carry no branches.
    float *sml = reinterpret_cast<float *>(&s_slot[0][0]);
    const int ns = a.n_split;
    const int n_ml = ns * G;
    const float2 *mlp = reinterpret_cast<const float2 *>(a.part_ml) + static_cast<size_t>(j) * n_ml;
    const bool merger = t < G * 32;
    const int h = merger ? t >> 5 : 0, d4 = (t & 31) * 4;
    const float4 *base = reinterpret_cast<const float4 *>(a.part_acc + (static_cast<size_t>(j) * ns * G + h) * 128 + d4);
    const size_t stride = static_cast<size_t>(G) * 32;              // float4 per split
    float4 ra[kAttnMergeRound], rb[kAttnMergeRound];
    auto load_round = [&](float4 (&r)[kAttnMergeRound], int s0) {
#pragma unroll
        for (int u = 0; u < kAttnMergeRound; ++u) r[u] = base[min(s0 + u, ns - 1) * stride];
    };
    // the first two pairs per thread go out first, then the first round of partials,
    // so the LDS stores of the pairs (and the barrier) wait for the pairs only
    const int ia = t, ib = kAttnThreads + t;
    const float2 va = mlp[min(ia, n_ml - 1)], vb = mlp[min(ib, n_ml - 1)];
    if (merger) load_round(ra, 0);
    if (ia < n_ml) { sml[2 * ia] = va.x; sml[2 * ia + 1] = va.y; }
    if (ib < n_ml) { sml[2 * ib] = vb.x; sml[2 * ib + 1] = vb.y; }
    for (int i = 2 * kAttnThreads + t; i < n_ml; i += kAttnThreads) {   // more pairs than 2 per thread
        const float2 v = mlp[i];
        sml[2 * i] = v.x;
        sml[2 * i + 1] = v.y;
    }
    __syncthreads();
    if (merger) {
        float M = -INFINITY;                // finite: split 0 holds token 0
        for (int s = 0; s < ns; ++s) M = fmaxf(M, sml[2 * (s * G + h)]);
        float L = 0.f, A0 = 0.f, A1 = 0.f, A2 = 0.f, A3 = 0.f;
        auto sum_round = [&](const float4 (&r)[kAttnMergeRound], int s0) {
#pragma unroll
            for (int u = 0; u < kAttnMergeRound; ++u) {
                const int s = min(s0 + u, ns - 1);
                const float f = s0 + u < ns ? exp2f(sml[2 * (s * G + h)] - M) : 0.f;   // 0 for empty splits too
                L += sml[2 * (s * G + h) + 1] * f;
                A0 += r[u].x * f; A1 += r[u].y * f; A2 += r[u].z * f; A3 += r[u].w * f;
            }
        };
        for (int s0 = 0; s0 < ns; s0 += 2 * kAttnMergeRound) {
            if (s0 + kAttnMergeRound < ns) load_round(rb, s0 + kAttnMergeRound);
            sum_round(ra, s0);
            if (s0 + kAttnMergeRound >= ns) break;
            if (s0 + 2 * kAttnMergeRound < ns) load_round(ra, s0 + 2 * kAttnMergeRound);
            sum_round(rb, s0 + kAttnMergeRound);
        }
        const float inv = 1.0f / L;
        uint16_t *o = a.out + (j * G + h) * 128 + d4;
        o[0] = f32_to_f16(A0 * inv);
        o[1] = f32_to_f16(A1 * inv);
        o[2] = f32_to_f16(A2 * inv);
        o[3] = f32_to_f16(A3 * inv);
    }
}

}  // namespace w4

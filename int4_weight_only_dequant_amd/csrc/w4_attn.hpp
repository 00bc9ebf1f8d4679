// Paged decode attention for gfx950: one query token, GQA, 16-token pages.
//
// The pages describe decode attention as softmax over q.K plus weighted-V
// accumulation, streamed over the KV cache page by page ("The Architecture of
// Modern Inference…", section "Three Critical Engineering Challenges", item 1;
// page size and the 4 KiB kv-head slice in "Building a Custom LLM Inference
// Runtime…", section "Technical Specifications and Hardware Alignment").
// Their Hopper design (one TMA producer warp, six consumer warps, mbarriers)
// is not used: here a work-group owns one kv head and a contiguous range of
// logical pages (split-KV).  Its 256 lanes cover one page per load: lane t
// holds token t / 16 of the page and dims 8 (t % 16) .. +7, so each lane
// reads 16 bytes of K and 16 bytes of V per page, and the 4 KiB slice of the
// page is one contiguous load per operand.  Those K and V registers serve all
// GQA query heads of the kv head.  Scores are reduced over the 16 lanes of a
// DPP row; each token slot keeps an online-softmax state (max, sum, 8 dims of
// the weighted V) per query head in fp32 (base-2 exponent domain).  At the
// end the 16 slots are merged through LDS, the work-group publishes its
// partial, and the last work-group of the kv head merges all splits and
// writes fp16 outputs.  Every barrier is reached by all waves (no barrier in
// lane- or wave-dependent control flow).  Partials are written with device-
// scope (sc1) stores; every wave waits for its stores to be acknowledged
// before the barrier that precedes the arrival atomic, so the last work-group
// never reads a partial before it is complete.
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

// Splits per kv head: about kAttnTargetSplits, each at least kAttnMinPps
// pages (a short split saves page-loop time but adds partials for the
// last-arriver merge to read).  Measured per call: context 640, at least 1,
// 2 or 4 pages per split 15.8, 12.4 and 12.6 us; context 8192 (512 pages),
// 32, 64 or 128 splits 27.9, 27.2 and 37.4 us.
#ifndef W4_ATTN_TARGET_SPLITS
#define W4_ATTN_TARGET_SPLITS 64
#endif
#ifndef W4_ATTN_MIN_PPS
#define W4_ATTN_MIN_PPS 2
#endif
constexpr int kAttnTargetSplits = W4_ATTN_TARGET_SPLITS;
constexpr int kAttnMinPps = W4_ATTN_MIN_PPS;
static_assert(kAttnTargetSplits >= 1 && kAttnTargetSplits <= 256 && kAttnMinPps >= 1, "attention split bounds");
inline int attn_pages_per_split(int n_pages_max) {
    const int pps = (n_pages_max + kAttnTargetSplits - 1) / kAttnTargetSplits;
    return pps < kAttnMinPps ? kAttnMinPps : pps;
}
inline int attn_n_split(int n_pages_max) {
    const int pps = attn_pages_per_split(n_pages_max);
    return (n_pages_max + pps - 1) / pps;
}

constexpr int kAttnChunk = 4;   // pages loaded together (8 x 16 B per lane)

// Arrival counters one 128-byte line apart: atomics on one line serialise
// (about 18 ns each), so with the kv heads' counters on one line the 4 x 64
// arrivals of a long context queued behind each other.
constexpr int kAttnCtrStride = 32;

template <int G>
__device__ __forceinline__ void attn_load_chunk(const AttnProblem &a, int j, int c0, int p_end, size_t lane_off,
                                                u32x4 (&k)[kAttnChunk], u32x4 (&v)[kAttnChunk]) {
    const size_t slice = static_cast<size_t>(kPage) * kHeadDim;
#pragma unroll
    for (int i = 0; i < kAttnChunk; ++i) {
        if (c0 + i < p_end) {
            const int phys = a.page_table[c0 + i];
            const size_t base = (static_cast<size_t>(phys) * a.n_kvh + j) * slice + lane_off;
            k[i] = *reinterpret_cast<const u32x4 *>(a.kpool + base);
            v[i] = *reinterpret_cast<const u32x4 *>(a.vpool + base);
        }
    }
}

template <int G>
__global__ __launch_bounds__(kThreads) void attn_decode_kernel(AttnProblem a) {
    __shared__ float s_m[16][G];
    __shared__ float s_l[16][G];
    __shared__ float s_acc[16][G][128];
    __shared__ int s_last;

    const int t = threadIdx.x;
    const int slot = t >> 4;          // token within the page
    const int dc = t & 15;            // 8-dim chunk
    const int j = blockIdx.x / a.n_split;
    const int sp = blockIdx.x % a.n_split;
    const int ctx = a.pos_ptr ? *a.pos_ptr + 1 : a.ctx;
    const int n_pages = (ctx + kPage - 1) / kPage;
    const int p_begin = sp * a.pages_per_split;
    int p_end = p_begin + a.pages_per_split;
    if (p_end > n_pages) p_end = n_pages;
    const size_t lane_off = static_cast<size_t>(slot) * kHeadDim + dc * 8;

    // issue the first chunk of K/V loads before anything else
    u32x4 kb[kAttnChunk], vb[kAttnChunk];
    attn_load_chunk<G>(a, j, p_begin, p_end, lane_off, kb, vb);

    // query heads of this kv head, 8 dims each
    uint32_t qv[G][4];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(a.q + (j * G + h) * 128 + dc * 8);
        qv[h][0] = v.x; qv[h][1] = v.y; qv[h][2] = v.z; qv[h][3] = v.w;
    }
    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
    }

    for (int c0 = p_begin; c0 < p_end; c0 += kAttnChunk) {
        u32x4 kc[kAttnChunk], vc[kAttnChunk];
#pragma unroll
        for (int i = 0; i < kAttnChunk; ++i) { kc[i] = kb[i]; vc[i] = vb[i]; }
        if (c0 + kAttnChunk < p_end)                      // prefetch the next chunk
            attn_load_chunk<G>(a, j, c0 + kAttnChunk, p_end, lane_off, kb, vb);
#pragma unroll
        for (int i = 0; i < kAttnChunk; ++i) {
            const int lp = c0 + i;
            if (lp >= p_end) break;                       // uniform across the work-group
            const int tok = lp * kPage + slot;
            float vf[8];
            vf[0] = static_cast<float>(as_h2(vc[i].x)[0]); vf[1] = static_cast<float>(as_h2(vc[i].x)[1]);
            vf[2] = static_cast<float>(as_h2(vc[i].y)[0]); vf[3] = static_cast<float>(as_h2(vc[i].y)[1]);
            vf[4] = static_cast<float>(as_h2(vc[i].z)[0]); vf[5] = static_cast<float>(as_h2(vc[i].z)[1]);
            vf[6] = static_cast<float>(as_h2(vc[i].w)[0]); vf[7] = static_cast<float>(as_h2(vc[i].w)[1]);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float sc = 0.f;
                sc = __builtin_amdgcn_fdot2(as_h2(qv[h][0]), as_h2(kc[i].x), sc, false);
                sc = __builtin_amdgcn_fdot2(as_h2(qv[h][1]), as_h2(kc[i].y), sc, false);
                sc = __builtin_amdgcn_fdot2(as_h2(qv[h][2]), as_h2(kc[i].z), sc, false);
                sc = __builtin_amdgcn_fdot2(as_h2(qv[h][3]), as_h2(kc[i].w), sc, false);
                sc = row16_sum(sc) * a.scale_log2;
                if (tok < ctx) {                          // uniform over the 16 lanes of a row
                    const float m_new = fmaxf(m[h], sc);
                    const float corr = exp2f(m[h] - m_new);   // 0 on the first token (m = -inf)
                    const float pw = exp2f(sc - m_new);
                    l[h] = l[h] * corr + pw;
#pragma unroll
                    for (int d = 0; d < 8; ++d) acc[h][d] = acc[h][d] * corr + pw * vf[d];
                    m[h] = m_new;
                }
            }
        }
    }

    // merge the 16 token slots of this work-group
#pragma unroll
    for (int h = 0; h < G; ++h) {
        if (dc == 0) { s_m[slot][h] = m[h]; s_l[slot][h] = l[h]; }
#pragma unroll
        for (int i = 0; i < 8; ++i) s_acc[slot][h][dc * 8 + i] = acc[h][i];
    }
    __syncthreads();
    const size_t pbase = (static_cast<size_t>(j) * a.n_split + sp) * G;
    for (int idx = t; idx < G * 128; idx += kThreads) {
        const int h = idx >> 7, d = idx & 127;
        float M = -INFINITY;
        for (int sl = 0; sl < 16; ++sl) M = fmaxf(M, s_m[sl][h]);
        float L = 0.f, A = 0.f;
        if (M != -INFINITY) {
            for (int sl = 0; sl < 16; ++sl) {
                const float f = exp2f(s_m[sl][h] - M);
                L += s_l[sl][h] * f;
                A += s_acc[sl][h][d] * f;
            }
        }
        store_agent(a.part_acc + (pbase + h) * 128 + d, A);
        if (d == 0) {
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
    // so no L2 holds a stale copy and plain 16-byte loads see them: up to 32
    // of them in flight per lane, where device-scope 4-byte loads took one
    // round trip per 8 splits.  The (max, sum) pairs go through LDS (reusing
    // s_acc, which holds them for n_split <= 1024); lane (h, 4 dims) then
    // streams its n_split float4 partials.
    float *sml = &s_acc[0][0][0];
    const int n_ml = a.n_split * G;
    const float2 *mlp = reinterpret_cast<const float2 *>(a.part_ml) + static_cast<size_t>(j) * n_ml;
    for (int i0 = 0; i0 < n_ml; i0 += 2 * kThreads) {             // (s, h) flattened
        const int ia = i0 + t, ib = i0 + kThreads + t;                // both loads in flight at once
        float2 va = make_float2(0.f, 0.f), vb = make_float2(0.f, 0.f);
        if (ia < n_ml) va = mlp[ia];
        if (ib < n_ml) vb = mlp[ib];
        if (ia < n_ml) { sml[2 * ia] = va.x; sml[2 * ia + 1] = va.y; }
        if (ib < n_ml) { sml[2 * ib] = vb.x; sml[2 * ib + 1] = vb.y; }
    }
    __syncthreads();
    if (t < G * 32) {
        const int h = t >> 5, d4 = (t & 31) * 4;
        float M = -INFINITY;
        for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, sml[2 * (s * G + h)]);
        float L = 0.f, A0 = 0.f, A1 = 0.f, A2 = 0.f, A3 = 0.f;
        const float4 *base =
            reinterpret_cast<const float4 *>(a.part_acc + (static_cast<size_t>(j) * a.n_split * G + h) * 128 + d4);
        const size_t stride = static_cast<size_t>(G) * 32;              // float4 per split
        for (int s0 = 0; s0 < a.n_split; s0 += 32) {
            float4 pa[32];
#pragma unroll
            for (int u = 0; u < 32; ++u)
                if (s0 + u < a.n_split) pa[u] = base[(s0 + u) * stride];
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                const int s = s0 + u;
                if (s < a.n_split) {
                    const float ms = sml[2 * (s * G + h)];
                    if (ms != -INFINITY) {
                        const float f = exp2f(ms - M);
                        L += sml[2 * (s * G + h) + 1] * f;
                        A0 += pa[u].x * f; A1 += pa[u].y * f; A2 += pa[u].z * f; A3 += pa[u].w * f;
                    }
                }
            }
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

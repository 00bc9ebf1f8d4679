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
// lane- or wave-dependent control flow), and the last-arriver exchange uses
// device-scope fences, so no work-group reads a partial before it is complete.
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
    unsigned *counter;          // [n_kvh]
    uint16_t *out;              // fp16 [n_qh][128]
};

inline int attn_pages_per_split(int n_pages_max) {
    int pps = (n_pages_max + 63) / 64;
    return pps < 2 ? 2 : pps;
}
inline int attn_n_split(int n_pages_max) {
    const int pps = attn_pages_per_split(n_pages_max);
    return (n_pages_max + pps - 1) / pps;
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

    const size_t slice = static_cast<size_t>(kPage) * kHeadDim;     // halves per kv-head slice
    const size_t lane_off = static_cast<size_t>(slot) * kHeadDim + dc * 8;
    u32x4 kn = {0, 0, 0, 0}, vn = {0, 0, 0, 0};
    if (p_begin < p_end) {
        const int phys = a.page_table[p_begin];
        const size_t base = (static_cast<size_t>(phys) * a.n_kvh + j) * slice + lane_off;
        kn = *reinterpret_cast<const u32x4 *>(a.kpool + base);
        vn = *reinterpret_cast<const u32x4 *>(a.vpool + base);
    }
    for (int lp = p_begin; lp < p_end; ++lp) {
        const u32x4 kc = kn, vc = vn;
        if (lp + 1 < p_end) {            // prefetch the next page of this split
            const int phys = a.page_table[lp + 1];
            const size_t base = (static_cast<size_t>(phys) * a.n_kvh + j) * slice + lane_off;
            kn = *reinterpret_cast<const u32x4 *>(a.kpool + base);
            vn = *reinterpret_cast<const u32x4 *>(a.vpool + base);
        }
        const int tok = lp * kPage + slot;
        float vf[8];
        vf[0] = static_cast<float>(as_h2(vc.x)[0]); vf[1] = static_cast<float>(as_h2(vc.x)[1]);
        vf[2] = static_cast<float>(as_h2(vc.y)[0]); vf[3] = static_cast<float>(as_h2(vc.y)[1]);
        vf[4] = static_cast<float>(as_h2(vc.z)[0]); vf[5] = static_cast<float>(as_h2(vc.z)[1]);
        vf[6] = static_cast<float>(as_h2(vc.w)[0]); vf[7] = static_cast<float>(as_h2(vc.w)[1]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float s = 0.f;
            s = __builtin_amdgcn_fdot2(as_h2(qv[h][0]), as_h2(kc.x), s, false);
            s = __builtin_amdgcn_fdot2(as_h2(qv[h][1]), as_h2(kc.y), s, false);
            s = __builtin_amdgcn_fdot2(as_h2(qv[h][2]), as_h2(kc.z), s, false);
            s = __builtin_amdgcn_fdot2(as_h2(qv[h][3]), as_h2(kc.w), s, false);
            s = row16_sum(s) * a.scale_log2;
            if (tok < ctx) {             // uniform over the 16 lanes of a row
                const float m_new = fmaxf(m[h], s);
                const float corr = exp2f(m[h] - m_new);   // 0 on the first token (m = -inf)
                const float pw = exp2f(s - m_new);
                l[h] = l[h] * corr + pw;
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[h][i] = acc[h][i] * corr + pw * vf[i];
                m[h] = m_new;
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
    __syncthreads();
    if (t < 64) {
        const bool last = arrive_last(a.counter + j, static_cast<unsigned>(a.n_split));
        if (t == 0) s_last = last ? 1 : 0;
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    // merge all splits of kv head j (fixed order: deterministic)
    for (int idx = t; idx < G * 128; idx += kThreads) {
        const int h = idx >> 7, d = idx & 127;
        float M = -INFINITY;
        for (int s = 0; s < a.n_split; ++s)
            M = fmaxf(M, load_agent(a.part_ml + ((static_cast<size_t>(j) * a.n_split + s) * G + h) * 2));
        float L = 0.f, A = 0.f;
        for (int s = 0; s < a.n_split; ++s) {
            const size_t pb = (static_cast<size_t>(j) * a.n_split + s) * G + h;
            const float ms = load_agent(a.part_ml + pb * 2);
            if (ms == -INFINITY) continue;
            const float f = exp2f(ms - M);
            L += load_agent(a.part_ml + pb * 2 + 1) * f;
            A += load_agent(a.part_acc + pb * 128 + d) * f;
        }
        a.out[(j * G + h) * 128 + d] = f32_to_f16(A / L);
    }
}

}  // namespace w4

// Streaming W4A16 GEMV for the standalone calls (w4a16_gemv, w4a16_mlp).
//
// Same arithmetic as w4_gemv_kernel (the pages' fp16-activation path,
// "Building a Custom LLM Inference Runtime for Qwen2.5-Coder-7B on NVIDIA H100
// Hopper Architecture", sections "Technical Specifications and Hardware
// Alignment" and "Engineering Challenges" item 3): nibbles become exact fp16
// integers in registers, v_dot2 products are summed in fp32 within a
// 128-element group, and the scaled group sums are accumulated in fp64.
//
// What differs is the mapping, chosen so that one launch streams the matrix
// at the HBM rate instead of paying a wave start-up per group:
// * The matrix is a row-major sequence of T tiles (64 packed rows x one
//   128-element K group = 4 KiB of codes + 128 B of scales).  The launch has
//   P work-groups (about 2 per CU, all resident); work-group B owns the
//   contiguous tile range [ceil(B T / P), ceil((B+1) T / P)), and its 4 waves
//   take every 4th tile of it with two tiles in flight (the next tile's loads
//   are issued before the current one is consumed).
// * Activations are read through the scalar cache (wave-uniform s_load), so
//   the activation operand of every dot product is an SGPR.  (Staging them
//   in LDS and reading 16-byte broadcasts instead measured 5% slower on the
//   gate+up shape.)
// * Per row block the waves' fp64 sums are added in wave order in LDS.  A row
//   block that lies inside one range gets its epilogue at once; otherwise
//   each owning work-group (consecutive ones) stores its sum in its own slot,
//   and the last to arrive adds the slots in slot order, runs the epilogue,
//   and zeroes the slots and the counter.  The summation order depends only
//   on the shape, so results are deterministic, and the workspace is all
//   zero again after every call: no clearing launch is needed.
#pragma once

#include "w4_gemv.hpp"

namespace w4 {

constexpr int kSgMaxRl = 8;          // row blocks one work-group's range may touch
#ifndef W4_SG_WG_TARGET
#define W4_SG_WG_TARGET 512
#endif
constexpr int kSgWgTarget = W4_SG_WG_TARGET;   // work-groups per launch (2 per CU)
// At least 8 tiles per work-group: on the 3584 x 3584 GEMV (1568 tiles) a
// call measured 8.4 us with 4 (392 work-groups), 7.7 with 8, 8.0 with 12 and
// 8.5 with 16: fewer work-groups share fewer row blocks, so fewer
// last-arriver reductions, until too few CUs stream.  Larger matrices keep
// kSgWgTarget work-groups either way.
#ifndef W4_SG_MIN_TILES
#define W4_SG_MIN_TILES 8
#endif
constexpr int kSgMinTiles = W4_SG_MIN_TILES;   // tiles per work-group below which P shrinks

struct SgProblem {
    const u32x4 *wq;          // packed codes
    const uint16_t *ws;       // packed scales
    const uint32_t *x;        // activations as fp16 pairs, K/2 words (int8: the activation buffer)
    uint32_t a8_scales, a8_sums;   // int8 activations: byte offsets of scales and sums in x
    int ng;                   // K / 128
    int T;                    // tiles = row blocks * ng
    int P;                    // work-groups
    int slot_stride;          // partial slots per shared row block
    int key_by_rb;            // shared row blocks keyed by row block (else by first owner)
    double *slots;            // [n_keys][slot_stride][64], zero between calls
    unsigned *ctr;            // [n_keys][kSgCtrStride] arrival counters, zero between calls
    unsigned *hdr;            // workspace mark: 0 (fresh) or kSgMark once used
};

// The workspace's first word: zero in a fresh workspace, set to kSgMark by
// the first call.  Any other value means memory that was never zeroed: the
// calls then write NaN outputs and leave the workspace alone instead of
// reducing through stale counters (cheap: one load per work-group, waited
// for only at the reduction).  Corruption of a zeroed workspace's counters
// is not detected.
constexpr unsigned kSgMark = 0x57344731u;
constexpr size_t kSgHdrBytes = 256;

// A row block shared by several work-groups is keyed by its index or by its
// first owner, whichever set is smaller (a work-group is the first owner of
// at most one shared row block: the one holding the end of its range).
struct SgGeom {
    int T, P, slot_stride, n_keys, key_by_rb;
};

// P: about kSgWgTarget work-groups, fewer for small matrices (at least
// kSgMinTiles tiles, one per wave, each), never more than one per tile, and
// enough that no range touches more than kSgMaxRl row blocks.  slot_stride bounds the
// work-groups that share one row block.
inline SgGeom sg_geom(int n_rb, int ng) {
    SgGeom g;
    g.T = n_rb * ng;
    const int64_t r_max = static_cast<int64_t>(kSgMaxRl - 1) * ng + 1;
    const int p_min = static_cast<int>((g.T + r_max - 1) / r_max);
    int P = kSgWgTarget;
    const int p_fill = (g.T + kSgMinTiles - 1) / kSgMinTiles;
    if (P > p_fill) P = p_fill;
    if (P < p_min) P = p_min;
    if (P > g.T) P = g.T;
    g.P = P;
    g.slot_stride = static_cast<int>((static_cast<int64_t>(ng - 1) * P) / g.T) + 2;
    g.key_by_rb = n_rb <= P;
    g.n_keys = g.key_by_rb ? n_rb : P;
    return g;
}

// Each counter on its own 128-byte line: atomics on one line serialise
// (about 18 ns each), and the shared row blocks of a small matrix all finish
// at about the same time.
constexpr int kSgCtrStride = 32;
inline size_t sg_ctr_bytes(const SgGeom &g) {
    return (static_cast<size_t>(g.n_keys) * kSgCtrStride * 4 + 255) & ~size_t(255);
}

// Workspace: the mark, the counters, then the slots.
inline size_t sg_ws_bytes(int n_rb, int ng) {
    const SgGeom g = sg_geom(n_rb, ng);
    return kSgHdrBytes + sg_ctr_bytes(g) + static_cast<size_t>(g.n_keys) * g.slot_stride * 64 * sizeof(double);
}

__device__ __forceinline__ int sg_range_begin(int B, int T, int P) {
    return static_cast<int>((static_cast<int64_t>(B) * T + P - 1) / P);
}
__device__ __forceinline__ int sg_owner(int t, int T, int P) {
    return static_cast<int>((static_cast<int64_t>(t) * P) / T);
}

__device__ __forceinline__ void sg_load(u32x4 (&w)[4], uint16_t &s, const SgProblem &p, int t) {
    const u32x4 *src = p.wq + static_cast<size_t>(t) * 256 + (threadIdx.x & 63);
#pragma unroll
    for (int c = 0; c < 4; ++c) w[c] = __builtin_nontemporal_load(src + c * 64);
    s = p.ws[static_cast<size_t>(t) * 64 + (threadIdx.x & 63)];
}

// One tile's scaled group sum, fp32 chained inside the group (as in
// w4_gemv_kernel).  Cheaper, but the chained accumulator's cut low bits add
// up: fine for O(1) activations, too coarse for large ones.
__device__ __forceinline__ double sg_tile(const u32x4 (&w)[4], uint16_t s, const_u32_ptr xg, uint32_t m_lo,
                                          uint32_t m_hi, uint32_t magic, uint32_t magic_hi) {
    float acc1 = 0.f, acc2 = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        dot8(w[c].x, xg + c * 16 + 0, acc1, acc2, m_lo, m_hi, magic, magic_hi);
        dot8(w[c].y, xg + c * 16 + 4, acc1, acc2, m_lo, m_hi, magic, magic_hi);
        dot8(w[c].z, xg + c * 16 + 8, acc1, acc2, m_lo, m_hi, magic, magic_hi);
        dot8(w[c].w, xg + c * 16 + 12, acc1, acc2, m_lo, m_hi, magic, magic_hi);
    }
    return static_cast<double>(acc1 + acc2) * static_cast<double>(f16_to_f32(s));
}

// One tile's scaled group sum from short 8-term sums added in fp64
// (dot8v_short), x from SGPRs.  The streaming GEMV's default: its x is any
// caller's vector (the MLP's down projection reads h of magnitude 10^2 and
// more), and the relative bound near outputs much smaller than their terms
// needs the short sums there (about 30% more VALU work per tile).
__device__ __forceinline__ double sg_tile_short(const u32x4 (&w)[4], uint16_t s, const_u32_ptr xg, uint32_t m_lo,
                                                uint32_t m_hi, uint32_t magic, uint32_t magic_hi) {
    double gs = 0.0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t ws4[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t xs[4] = {xg[c * 16 + j * 4 + 0], xg[c * 16 + j * 4 + 1], xg[c * 16 + j * 4 + 2],
                                    xg[c * 16 + j * 4 + 3]};
            gs += static_cast<double>(dot8v_short(ws4[j], xs, m_lo, m_hi, magic, magic_hi));
        }
    }
    return gs * static_cast<double>(f16_to_f32(s));
}

// ---------------------------------------------------------------------------
// Int8 activations (the pages' integer path: "Building a Custom LLM Inference
// Runtime…", section "Engineering Challenges" item 3, and "The Architecture of
// Modern Inference…", section "Three Critical Engineering Challenges" item 3).
// The fp16 activations are quantised by a separate kernel, per group of 128
// along K: scale s = max|x| / 127 in fp32, codes round-half-even(x / s) in
// fp32, clamped to [-127, 127] (scale 0 and zero codes for an all-zero group).
// Activation buffer (device, w4a8_act_bytes(K) bytes):
//   [0, K)            int8 codes; each block of 8 elements e0..e7 is stored as
//                     two words (e0, e4, e1, e5), (e2, e6, e3, e7), matching the
//                     bytes (w & 0x0F0F0F0F) and ((w >> 4) & 0x0F0F0F0F) of a
//                     packed weight word (e0 e2 e4 e6 in the low half-word,
//                     e1 e3 e5 e7 in the high half-word);
//   [A, A + K/32)     fp32 scales, A = K rounded up to 256;
//   [B, B + K/32)     int32 sums of each group's codes, B = A + (K/32 rounded
//                     up to 256).
// A group's integer dot product sum_k (u_k - 8) c_k = sum_k u_k c_k - 8 sum_k c_k
// (u = q + 8, the stored nibble) runs on v_dot4_i32_i8: two of them per packed
// word, four bytes each, exact in int32.  Scaled by s_w * s_x in fp64 it is
// exact (11 + 24 + 18 bits), and the groups are added in fp64.

inline size_t a8_scales_off(int64_t K) { return static_cast<size_t>((K + 255) & ~int64_t(255)); }
inline size_t a8_sums_off(int64_t K) { return a8_scales_off(K) + ((static_cast<size_t>(K / 128) * 4 + 255) & ~size_t(255)); }
inline size_t a8_act_bytes(int64_t K) { return a8_sums_off(K) + static_cast<size_t>(K / 128) * 4; }

// One wave per group of 128 activations; lane l quantises elements 2l, 2l+1.
__global__ __launch_bounds__(64) void a8_quantize_kernel(const uint16_t *x, int8_t *codes, float *scales,
                                                         int *sums) {
    const int g = blockIdx.x, lane = threadIdx.x;
    const uint32_t pair = reinterpret_cast<const uint32_t *>(x + static_cast<size_t>(g) * 128)[lane];
    const float v0 = f16_to_f32(static_cast<uint16_t>(pair & 0xFFFFu));
    const float v1 = f16_to_f32(static_cast<uint16_t>(pair >> 16));
    float amax = fmaxf(fabsf(v0), fabsf(v1));
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float sc = amax / 127.0f;                 // IEEE division, rounded to nearest even
    int c0 = 0, c1 = 0;
    if (sc != 0.0f) {
        c0 = static_cast<int>(fminf(fmaxf(rintf(v0 / sc), -127.0f), 127.0f));
        c1 = static_cast<int>(fminf(fmaxf(rintf(v1 / sc), -127.0f), 127.0f));
    }
    int sum = c0 + c1;
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    // element e of the group: block e / 8, position p = e % 8 -> byte
    // 8 (e / 8) + 4 ((p >> 1) & 1) + ((p >> 2) & 1) + 2 (p & 1)
    int8_t *cg = codes + static_cast<size_t>(g) * 128;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int e = 2 * lane + u, pp = e & 7;
        cg[(e & ~7) + 4 * ((pp >> 1) & 1) + ((pp >> 2) & 1) + 2 * (pp & 1)] = static_cast<int8_t>(u ? c1 : c0);
    }
    if (lane == 0) {
        scales[g] = sc;
        sums[g] = sum;
    }
}

// One tile's scaled group sum with int8 activations: xg = the group's 32
// code words, sx its scale, sumc the sum of its codes.
__device__ __forceinline__ double sg_tile_a8(const u32x4 (&w)[4], uint16_t s, const_u32_ptr xg, float sx,
                                             int sumc) {
    int acc = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t ws4[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int b = c * 4 + i;                 // block of 8 elements within the group
            const int lo = static_cast<int>(ws4[i] & 0x0F0F0F0Fu), hi = static_cast<int>((ws4[i] >> 4) & 0x0F0F0F0Fu);
            acc = __builtin_amdgcn_sdot4(lo, static_cast<int>(xg[2 * b]), acc, false);
            acc = __builtin_amdgcn_sdot4(hi, static_cast<int>(xg[2 * b + 1]), acc, false);
        }
    }
    const int dot = acc - 8 * sumc;
    return static_cast<double>(f16_to_f32(s)) * static_cast<double>(sx) * static_cast<double>(dot);
}

// kShort: short 8-term sums added in fp64 (sg_tile_short); off only where
// the activations are O(1) by construction (the MLP's normalised gate/up
// input), which takes one fp32 chain per group.
template <class Epi, bool kA8 = false, bool kShort = true>
__global__ __launch_bounds__(kThreads) void sg_gemv_kernel(SgProblem p, Epi epi) {
    __shared__ double red[kSgMaxRl * 256];
    const int B = blockIdx.x;
    const unsigned mark = load_agent(p.hdr);   // used at the reduction
    if (B == 0 && threadIdx.x == 0 && mark == 0u) store_agent(p.hdr, kSgMark);
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int t_begin = sg_range_begin(B, p.T, p.P), t_end = sg_range_begin(B + 1, p.T, p.P);
    const int rb0 = t_begin / p.ng;
    const int n_rl = (t_end - 1) / p.ng - rb0 + 1;
    // each thread clears the slots it later writes (rl, its wave, its lane)
    for (int i = threadIdx.x; i < n_rl * 256; i += kThreads) red[i] = 0.0;

    const uint32_t m_lo = vreg_const(0x000F000Fu), m_hi = vreg_const(0x00F000F0u), magic = vreg_const(0x64006400u), magic_hi = vreg_const(0x54005400u);
    const const_u32_ptr xc = as_const(p.x);
    u32x4 wa[4], wb[4];
    uint16_t sa = 0, sb = 0;
    int t = t_begin + wave;
    if (t < t_end) sg_load(wa, sa, p, t);
    int cur = -1;
    double acc = 0.0;
    auto consume = [&](const u32x4 (&w)[4], uint16_t s, int tt) {
        const int rbt = tt / p.ng;
        const int g = tt - rbt * p.ng;
        const int rl = rbt - rb0;
        if (rl != cur) {
            if (cur >= 0) red[cur * 256 + wave * 64 + lane] = acc;
            acc = 0.0;
            cur = rl;
        }
        if constexpr (kA8) {
            const const_u32_ptr aux = as_const(p.x);
            acc += sg_tile_a8(w, s, xc + g * 32, __builtin_bit_cast(float, aux[p.a8_scales / 4 + g]),
                              static_cast<int>(aux[p.a8_sums / 4 + g]));
        } else {
            if constexpr (kShort)
                acc += sg_tile_short(w, s, xc + g * 64, m_lo, m_hi, magic, magic_hi);
            else
                acc += sg_tile(w, s, xc + g * 64, m_lo, m_hi, magic, magic_hi);
        }
    };
    while (t < t_end) {
        if (t + 4 < t_end) sg_load(wb, sb, p, t + 4);
        consume(wa, sa, t);
        t += 4;
        if (t >= t_end) break;
        if (t + 4 < t_end) sg_load(wa, sa, p, t + 4);
        consume(wb, sb, t);
        t += 4;
    }
    if (cur >= 0) red[cur * 256 + wave * 64 + lane] = acc;
    __syncthreads();

    // one wave per row block of the range
    const bool dirty = __builtin_amdgcn_readfirstlane(mark) != 0u && __builtin_amdgcn_readfirstlane(mark) != kSgMark;
    for (int rl = wave; rl < n_rl; rl += 4) {
        const double *rr = red + rl * 256 + lane;
        const double v = ((rr[0] + rr[64]) + rr[128]) + rr[192];
        const int rb = rb0 + rl;
        const int a = rb * p.ng;
        const int row = rb * 64 + lane;
        if (dirty) {   // a workspace that was never zeroed: visible failure
            epi(row, lane, __builtin_nan(""));
            continue;
        }
        if (a >= t_begin && a + p.ng <= t_end) {
            epi(row, lane, v);
            continue;
        }
        const int first = sg_owner(a, p.T, p.P);
        const int n_c = sg_owner(a + p.ng - 1, p.T, p.P) - first + 1;
        const int key = p.key_by_rb ? rb : first;
        double *base = p.slots + static_cast<size_t>(key) * p.slot_stride * 64 + lane;
        store_agent(base + (B - first) * 64, v);
        if (!arrive_last(p.ctr + static_cast<size_t>(key) * kSgCtrStride, static_cast<unsigned>(n_c))) continue;
        // all slots in parallel, summed in slot order, then cleared
        double tot = 0.0;
        int k = 0;
        for (; k + 8 <= n_c; k += 8) {
            double s8[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) s8[u] = load_agent(base + (k + u) * 64);
#pragma unroll
            for (int u = 0; u < 8; ++u) tot += s8[u];
        }
        for (; k < n_c; ++k) tot += load_agent(base + k * 64);
        for (k = 0; k < n_c; ++k) store_agent(base + k * 64, 0.0);
        epi(row, lane, tot);
    }
}

}  // namespace w4

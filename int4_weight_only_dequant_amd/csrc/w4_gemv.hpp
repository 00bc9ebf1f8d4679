// W4A16 and fp16 GEMV kernels for gfx950 (batch 1, one output row per lane).
//
// The quantised projections are symmetric group-wise int4 with group 128 and
// one fp16 scale per group, multiplied with fp16 activations (the pages'
// fp16-activation path: "Building a Custom LLM Inference Runtime for
// Qwen2.5-Coder-7B on NVIDIA H100 Hopper Architecture", sections "Technical
// Specifications and Hardware Alignment" and "Engineering Challenges" item 3).
//
// Mapping: a work-group of 4 waves owns one block of 64 packed rows (lane l of
// every wave holds row 64 b + l) and a contiguous range of K groups; the waves
// stride over that range.  Per group a lane issues four 16-byte loads (each
// wave load is one contiguous KiB of the packed stream) and the wave reads the
// group's 128 activations once through the scalar cache (s_load), so the
// activation operand of every dot product is an SGPR.  Batch-1 GEMV is a
// vector-matrix product with one use per weight, so there is no MFMA here:
// the VALU turns nibbles into fp16 (mask + OR an exponent + subtract) and
// v_dot2c_f32_f16 accumulates.  Every product q*x is exact in fp32; a
// group's sum of 128 of them rounds in fp32 (relative to the magnitude of its
// terms, about 2^-24 per addition), and across groups the scaled sums are
// accumulated in fp64.  Work-groups that split one row
// block along K publish fp64 partials, and the last to arrive sums them in a
// fixed order and runs the epilogue, so results are deterministic.
#pragma once

#include "w4_device.hpp"

namespace w4 {

struct W4Problem {
    const u32x4 *wq;      // packed codes
    const uint16_t *ws;   // packed scales
    const uint32_t *x;    // activations as fp16 pairs, K/2 words
    int n_groups;         // K / 128
    int n_rb;             // row blocks
    int n_split;          // work-groups per row block along K
    double *partial;      // [n_split][n_rb * 64] (n_split > 1)
    unsigned *counter;    // [n_rb][kGemvCtrStride], zero between calls
};

// One 128-byte line per row block's arrival counter: atomics on one line
// serialise, and the split-K work-groups of many row blocks arrive together.
constexpr int kGemvCtrStride = 32;

// 8 weights of one 32-bit word against 4 activation pairs.  Word layout:
// element 2j in bits [4j, 4j+4), element 2j+1 in bits [16+4j, 16+4j+4),
// stored as u = q + 8.  (w & 0x000F000F) | 0x6400_6400 is the fp16 pair
// (1024 + u0, 1024 + u1): the nibble lands on the mantissa bits of weight 1
// under exponent 2^10, and subtracting 1032 gives (q0, q1) exactly.  The
// nibbles at bits 4..7 sit on mantissa bits of weight 16 under 2^10, so they
// are OR-ed under exponent 2^6 instead ((w & 0x00F000F0) | 0x5400_5400 =
// 64 + u, minus 72 gives q).  Every product q x is exact in fp32.
//
// dot8 / dot8v accumulate the 8 products into an fp32 accumulator with
// v_dot2c_f32_f16 (13 VALU operations per 8 weights).  That instruction does
// not round correctly: the low bits of its accumulator operand are cut where
// the sum is formed (measured on gfx950: 0.7% of random sums off by more than
// half an ulp, up to about one ulp), so a long chain drifts by about 3 times
// the error of correctly rounded fp32 sums.
__device__ __forceinline__ void dot8(uint32_t w, const_u32_ptr xs, float &acc1, float &acc2, uint32_t m_lo,
                                     uint32_t m_hi, uint32_t magic, uint32_t magic_hi) {
    const h2 k1032 = {static_cast<_Float16>(1032.0f), static_cast<_Float16>(1032.0f)};
    const h2 k72 = {static_cast<_Float16>(72.0f), static_cast<_Float16>(72.0f)};
    const uint32_t w8 = w >> 8;
    const h2 q01 = as_h2((w & m_lo) | magic) - k1032;
    const h2 q23 = as_h2((w & m_hi) | magic_hi) - k72;
    const h2 q45 = as_h2((w8 & m_lo) | magic) - k1032;
    const h2 q67 = as_h2((w8 & m_hi) | magic_hi) - k72;
    acc1 = __builtin_amdgcn_fdot2(q01, as_h2(xs[0]), acc1, false);
    acc2 = __builtin_amdgcn_fdot2(q23, as_h2(xs[1]), acc2, false);
    acc1 = __builtin_amdgcn_fdot2(q45, as_h2(xs[2]), acc1, false);
    acc2 = __builtin_amdgcn_fdot2(q67, as_h2(xs[3]), acc2, false);
}

// Same as dot8 with the 4 activation pairs in VGPRs (broadcast LDS reads).
__device__ __forceinline__ void dot8v(uint32_t w, const uint32_t (&xs)[4], float &acc1, float &acc2,
                                      uint32_t m_lo, uint32_t m_hi, uint32_t magic, uint32_t magic_hi) {
    const h2 k1032 = {static_cast<_Float16>(1032.0f), static_cast<_Float16>(1032.0f)};
    const h2 k72 = {static_cast<_Float16>(72.0f), static_cast<_Float16>(72.0f)};
    const uint32_t w8 = w >> 8;
    const h2 q01 = as_h2((w & m_lo) | magic) - k1032;
    const h2 q23 = as_h2((w & m_hi) | magic_hi) - k72;
    const h2 q45 = as_h2((w8 & m_lo) | magic) - k1032;
    const h2 q67 = as_h2((w8 & m_hi) | magic_hi) - k72;
    acc1 = __builtin_amdgcn_fdot2(q01, as_h2(xs[0]), acc1, false);
    acc2 = __builtin_amdgcn_fdot2(q23, as_h2(xs[1]), acc2, false);
    acc1 = __builtin_amdgcn_fdot2(q45, as_h2(xs[2]), acc1, false);
    acc2 = __builtin_amdgcn_fdot2(q67, as_h2(xs[3]), acc2, false);
}

// A pair sum a.x b.x + a.y b.y from a zero accumulator: correctly rounded
// (the same measurement: every sum but 13 in 2^20 random ones).  Kept as the
// builtin, not an asm dot: the compiler then spaces a dot's result from its
// reader by the wait states the hardware needs, which it cannot do for an
// instruction hidden in asm (an asm dot read one instruction later returned
// the previous contents of its destination).
__device__ __forceinline__ float dot2z(h2 a, h2 b) { return __builtin_amdgcn_fdot2(a, b, 0.0f, false); }

// The 8 products of dot8v as one short sum for the caller to add in fp64: two
// 4-term chains (a pair sum from zero, then one accumulating dot) added with
// an IEEE fp32 add.  The accumulator's truncation then touches one addition
// per 4 terms instead of a whole group's chain, so a group's error stays at
// the rounding of 8-term sums, unbiased in practice.  Used where activations
// are large (SwiGLU output of 10^2 and more, any caller's vector in the
// standalone GEMV), so that outputs near zero stay within the GEMV tolerance:
// 18 VALU operations per 8 weights instead of 13 (each chain needs its zeroed
// accumulator; the fp64 conversion and add).  Four correctly rounded pair
// sums added in fp32 halved the worst layer-test error and cost 2.4% more per
// decode step.  Contraction is off here: with it the compiler folds the final
// add into a chained accumulation.
__device__ __forceinline__ float dot8v_short(uint32_t w, const uint32_t (&xs)[4], uint32_t m_lo, uint32_t m_hi,
                                             uint32_t magic, uint32_t magic_hi) {
#pragma clang fp contract(off)
    const h2 k1032 = {static_cast<_Float16>(1032.0f), static_cast<_Float16>(1032.0f)};
    const h2 k72 = {static_cast<_Float16>(72.0f), static_cast<_Float16>(72.0f)};
    const uint32_t w8 = w >> 8;
    const h2 q01 = as_h2((w & m_lo) | magic) - k1032;
    const h2 q23 = as_h2((w & m_hi) | magic_hi) - k72;
    const h2 q45 = as_h2((w8 & m_lo) | magic) - k1032;
    const h2 q67 = as_h2((w8 & m_hi) | magic_hi) - k72;
    const float pa = __builtin_amdgcn_fdot2(q45, as_h2(xs[2]), dot2z(q01, as_h2(xs[0])), false);
    const float pb = __builtin_amdgcn_fdot2(q67, as_h2(xs[3]), dot2z(q23, as_h2(xs[1])), false);
    return pa + pb;
}

// Sum over the work-group's 4 waves of one fp64 value per lane; result valid
// in wave 0.
__device__ __forceinline__ double wg_sum4(double v, double *lds) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    lds[wave * 64 + lane] = v;
    __syncthreads();
    double t = 0;
    if (wave == 0) t = ((lds[lane] + lds[64 + lane]) + lds[128 + lane]) + lds[192 + lane];
    return t;
}

template <class Epi>
__global__ __launch_bounds__(kThreads) void w4_gemv_kernel(W4Problem p, Epi epi) {
    __shared__ double red[4 * 64];
    __shared__ int s_flag;
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int rb = blockIdx.x % p.n_rb;
    const int sp = blockIdx.x / p.n_rb;
    const int g_begin = static_cast<int>((static_cast<int64_t>(sp) * p.n_groups) / p.n_split);
    const int g_end = static_cast<int>((static_cast<int64_t>(sp + 1) * p.n_groups) / p.n_split);

    const u32x4 *wq = p.wq + static_cast<size_t>(rb) * p.n_groups * 4 * 64 + lane;
    const uint16_t *ws = p.ws + static_cast<size_t>(rb) * p.n_groups * 64 + lane;
    const uint32_t m_lo = vreg_const(0x000F000Fu), m_hi = vreg_const(0x00F000F0u),
                   magic = vreg_const(0x64006400u), magic_hi = vreg_const(0x54005400u);

    double acc = 0.0;
    for (int g = g_begin + wave; g < g_end; g += 4) {
        u32x4 v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = __builtin_nontemporal_load(wq + (g * 4 + c) * 64);
        const uint16_t sbits = ws[g * 64];
        const const_u32_ptr xg = as_const(p.x) + g * 64;
        float acc1 = 0.f, acc2 = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            dot8(v[c].x, xg + c * 16 + 0, acc1, acc2, m_lo, m_hi, magic, magic_hi);
            dot8(v[c].y, xg + c * 16 + 4, acc1, acc2, m_lo, m_hi, magic, magic_hi);
            dot8(v[c].z, xg + c * 16 + 8, acc1, acc2, m_lo, m_hi, magic, magic_hi);
            dot8(v[c].w, xg + c * 16 + 12, acc1, acc2, m_lo, m_hi, magic, magic_hi);
        }
        acc += static_cast<double>(acc1 + acc2) * static_cast<double>(f16_to_f32(sbits));
    }

    double total = wg_sum4(acc, red);
    const int row = rb * 64 + lane;
    if (p.n_split > 1) {
        // publish this split's partial; the last work-group of the row block
        // sums all of them (all 4 waves load in parallel, fixed order)
        const size_t n_rows = static_cast<size_t>(p.n_rb) * 64;
        if (wave == 0) {
            store_agent(p.partial + sp * n_rows + row, total);
            const bool last = arrive_last(p.counter + static_cast<size_t>(rb) * kGemvCtrStride,
                                          static_cast<unsigned>(p.n_split));
            if (lane == 0) s_flag = last ? 1 : 0;
        }
        __syncthreads();
        if (!s_flag) return;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        double part = 0.0;
        int s = wave;
        for (; s + 12 < p.n_split; s += 16) {
            const double a0 = load_agent(p.partial + s * n_rows + row);
            const double a1 = load_agent(p.partial + (s + 4) * n_rows + row);
            const double a2 = load_agent(p.partial + (s + 8) * n_rows + row);
            const double a3 = load_agent(p.partial + (s + 12) * n_rows + row);
            part += a0;
            part += a1;
            part += a2;
            part += a3;
        }
        for (; s < p.n_split; s += 4) part += load_agent(p.partial + s * n_rows + row);
        total = wg_sum4(part, red);
    }
    if (wave == 0) epi(row, lane, total);
    if constexpr (Epi::kGridTail) epi.grid_tail(p.n_rb, s_flag);
}

// ---------------------------------------------------------------- epilogues --
// Called by all 64 lanes of one wave with (packed row, lane, fp64 result).

struct EpiStoreF16 {          // y[row] = fp16(v)
    static constexpr bool kGridTail = false;
    uint16_t *y;
    int n;
    __device__ void operator()(int row, int, double v) const {
        if (row < n) y[row] = f64_to_f16(v);
    }
};

struct EpiResidual {          // x[row] += v   (fp64 residual stream)
    static constexpr bool kGridTail = false;
    double *x;
    int n;
    __device__ void operator()(int row, int, double v) const {
        if (row < n) x[row] += v;
    }
};

// Residual update followed by the RMSNorm that feeds the next GEMV:
// x[row] += v; then, once every row block is done, the last work-group to
// finish computes a = fp16(x / sqrt(mean(x^2) + eps) * w) for all of x.
// Each row block publishes the sum of squares of its 64 new values; the
// grand total is summed in row-block order, so results are deterministic.
struct EpiResidualNorm {
    static constexpr bool kGridTail = true;
    double *x;
    int n;
    const uint16_t *w;        // norm weight [n]
    uint16_t *a;              // fp16 output [n]
    double *ss;               // [n_rb] sums of squares
    unsigned *counter;        // arrivals of row blocks (zero between calls)
    double eps;
    __device__ void operator()(int row, int lane, double v) const {
        double xn = 0.0;
        if (row < n) {
            xn = x[row] + v;
            store_agent(x + row, xn);
        }
        double sq = xn * xn;
        for (int off = 32; off >= 1; off >>= 1) sq += __shfl_xor(sq, off);
        if (lane == 0) store_agent(ss + (row >> 6), sq);
    }
    // all 4 waves; block_last = whether this work-group ran the epilogue
    __device__ void grid_tail(int n_rb, int &flag) const {
        __shared__ double s_rms;
        const int t = threadIdx.x;
        if (t < 64) {
            const bool last = arrive_last(counter, static_cast<unsigned>(n_rb));
            if (t == 0) flag = last ? 1 : 0;
        }
        __syncthreads();
        if (!flag) return;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        if (t < 64) {
            double tot = 0.0;
            for (int b = 0; b < n_rb; ++b) tot += load_agent(ss + b);   // fixed order
            if (t == 0) s_rms = sqrt(tot / n + eps);
        }
        __syncthreads();
        const double r = s_rms;
        for (int i = t; i < n; i += kThreads)
            a[i] = f64_to_f16(load_agent(x + i) / r * static_cast<double>(f16_to_f32(w[i])));
    }
};

// gate/up interleaved rows: even lane holds gate_i, odd lane up_i;
// h[i] = fp16(silu(gate_i) * up_i).
struct EpiSwiGLU {
    static constexpr bool kGridTail = false;
    uint16_t *h;
    int n_pairs;
    __device__ void operator()(int row, int lane, double v) const {
        const double other = shfl_xor1(v);
        if ((lane & 1) == 0 && (row >> 1) < n_pairs) {
            const double g = v, u = other;
            h[row >> 1] = f64_to_f16(g / (1.0 + exp(-g)) * u);
        }
    }
};

// QKV rows in rotary-pair order (packed row 2i of a head = dim i, 2i+1 = dim
// i+64): adds the bias, rotates q and k heads by the position's angles, rounds
// to fp16, writes q to qbuf and k, v to the paged cache slot of the position.
struct EpiQKV {
    static constexpr bool kGridTail = false;
    const uint16_t *bias;     // fp16 [rows], logical order
    const double *rope;       // [max_pos][64][2] = (cos, sin)
    const int *pos_ptr;       // current position
    const int *page_table;    // logical page -> physical page
    uint16_t *qbuf;           // fp16 [n_qh * 128]
    uint16_t *kcache;         // this layer's K pool [pages][n_kvh][16][128]
    uint16_t *vcache;
    int n_qh, n_kvh;
    __device__ void operator()(int row, int lane, double v) const {
        const int head = row >> 7;
        const int i = (row & 127) >> 1;
        const int hi = row & 1;
        const int dim = i + 64 * hi;
        const int logical = head * 128 + dim;
        v += static_cast<double>(f16_to_f32(bias[logical]));
        const double partner = shfl_xor1(v);
        const int pos = *pos_ptr;
        double out = v;
        if (head < n_qh + n_kvh) {
            const double c = rope[(static_cast<size_t>(pos) * 64 + i) * 2];
            const double s = rope[(static_cast<size_t>(pos) * 64 + i) * 2 + 1];
            out = hi ? partner * s + v * c : v * c - partner * s;
        }
        const uint16_t h16 = f64_to_f16(out);
        if (head < n_qh) {
            qbuf[logical] = h16;
        } else {
            const int kv = head - n_qh;
            const int j = kv < n_kvh ? kv : kv - n_kvh;
            const int phys = page_table[pos >> 4];
            const size_t off = ((static_cast<size_t>(phys) * n_kvh + j) * kPage + (pos & 15)) * kHeadDim + dim;
            (kv < n_kvh ? kcache : vcache)[off] = h16;
        }
    }
};

// ------------------------------------------------------- fp16 lm_head GEMV --
// Packed fp16 rows (16 bytes = 8 elements per lane per chunk), fp32
// accumulation; writes fp32 logits and folds the greedy choice into one
// 64-bit atomic max of (order-preserving float bits, ~index): the largest
// logit wins and, among equal logits, the lowest index.

__device__ __forceinline__ uint64_t argmax_key(float v, int idx) {
    uint32_t u = __float_as_uint(v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (static_cast<uint64_t>(u) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(idx));
}

struct F16Problem {
    const u32x4 *w;       // packed fp16 rows
    const uint32_t *x;    // fp16 pairs, K/2 words
    int n_chunks;         // K / 8
    int n_rb;
    int n;                // valid rows
    float *out;           // fp32 [n]
    unsigned long long *best;  // argmax key (nullptr: skip)
};

__global__ __launch_bounds__(kThreads) void f16_gemv_kernel(F16Problem p) {
    __shared__ float red[4 * 64];
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int rb = blockIdx.x;
    const int c_begin = (p.n_chunks * wave) / 4, c_end = (p.n_chunks * (wave + 1)) / 4;
    const u32x4 *w = p.w + static_cast<size_t>(rb) * p.n_chunks * 64 + lane;
    float acc0 = 0.f, acc1 = 0.f;
    int c = c_begin;
    for (; c + 8 <= c_end; c += 8) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(w + (c + u) * 64);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const const_u32_ptr xs = as_const(p.x) + (c + u) * 4;
            acc0 = __builtin_amdgcn_fdot2(as_h2(v[u].x), as_h2(xs[0]), acc0, false);
            acc1 = __builtin_amdgcn_fdot2(as_h2(v[u].y), as_h2(xs[1]), acc1, false);
            acc0 = __builtin_amdgcn_fdot2(as_h2(v[u].z), as_h2(xs[2]), acc0, false);
            acc1 = __builtin_amdgcn_fdot2(as_h2(v[u].w), as_h2(xs[3]), acc1, false);
        }
    }
    for (; c < c_end; ++c) {
        const u32x4 v = __builtin_nontemporal_load(w + c * 64);
        const const_u32_ptr xs = as_const(p.x) + c * 4;
        acc0 = __builtin_amdgcn_fdot2(as_h2(v.x), as_h2(xs[0]), acc0, false);
        acc1 = __builtin_amdgcn_fdot2(as_h2(v.y), as_h2(xs[1]), acc1, false);
        acc0 = __builtin_amdgcn_fdot2(as_h2(v.z), as_h2(xs[2]), acc0, false);
        acc1 = __builtin_amdgcn_fdot2(as_h2(v.w), as_h2(xs[3]), acc1, false);
    }
    red[threadIdx.x] = acc0 + acc1;
    __syncthreads();
    if (wave != 0) return;
    const float logit = ((red[lane] + red[64 + lane]) + red[128 + lane]) + red[192 + lane];
    const int row = rb * 64 + lane;
    if (row < p.n) p.out[row] = logit;
    if (!p.best) return;
    uint64_t key = row < p.n ? argmax_key(logit, row) : 0;
    for (int off = 32; off >= 1; off >>= 1) {
        const uint64_t o = __shfl_xor(key, off);
        key = o > key ? o : key;
    }
    if (lane == 0) atomicMax(p.best, static_cast<unsigned long long>(key));
}

// Split-K policy: aim for ~2048 work-groups (8 per CU), at least one group per
// wave in every work-group.
inline int gemv_split(int n_rb, int n_groups) {
    int s = (2048 + n_rb / 2) / n_rb;
    const int max_s = n_groups / 4 > 0 ? n_groups / 4 : 1;
    if (s > max_s) s = max_s;
    if (s < 1) s = 1;
    return s;
}

}  // namespace w4

// Prompt prefill on gfx950 matrix cores: the W4A16 GEMM (M tokens at once),
// causal paged attention over the prompt chunk and the cache before it, and
// the per-token glue of a layer.
//
// The pages give the time to first token of a 512-token prompt without
// describing the prefill itself (performance comparison table under
// "Technical Specifications and Benchmarking Data" of "The Architecture of
// Modern Inference: A Deep Dive into the Development of the Annotated LLM
// Runtime for NVIDIA Hopper GPUs"; "Summary" of "How To Build Your Own LLM
// Runtime From Scratch").  The arithmetic here is that of the decode step applied to M
// positions: the same projections, norms, RoPE, SwiGLU and fp16 storage
// points, with position p attending to positions 0..p.
#pragma once

#include "w4_device.hpp"

namespace w4 {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPrefillMax = W4_PREFILL_MAX;   // tokens per prefill call
constexpr int kGemmBM = 128;         // tokens per GEMM work-group (and per wave)

// ------------------------------------------------------------ W4A16 GEMM --
//
// out[s][m][n] = sum over the groups g of split s of
//                s[n][g] * sum_{k in g} x[m][k] * q[n][k]
//
// A work-group computes 128 tokens x 128 packed rows (4 waves, each all 128
// tokens x 32 rows, so every dequantised weight operand feeds 4 MFMAs) over
// the groups of its split.  Per group of 128 K:
//  - the 128 x 128 activation tile is staged in LDS by direct global->LDS
//    loads (16 bytes per lane, double-buffered, one group ahead); the 16-byte
//    chunk c of row r sits at chunk c ^ (r % 16) of its LDS row, so that the
//    operand reads of 16 consecutive rows at one chunk hit distinct banks;
//  - each wave loads its row block's codes for the group straight into
//    registers (one group ahead) in the packer's lane layout, and turns them
//    into exact small-integer fp16 operands;
//  - 8 MFMA 32x32x16 steps per 32x32 output tile accumulate the group's
//    integer dot products in fp32 from zero (each product is exact), and the
//    group's fp16 scale is applied once per output while adding into an fp64
//    accumulator: fp32 within a group, fp64 across groups, as in the GEMV.
// Operand k order: for MFMA step t and lane half hf = lane / 32, the 8
// consecutive elements k = 64 hf + 8 t + e (e = 0..7) of the group.  Both
// operands use the same order, so the contraction is over all 128 k.
// The lane's B slice for step t is word t of the two 16-byte code slots of
// chunks 4g + 2 hf and 4g + 2 hf + 1 of its row: one 16-byte load per slot.

struct GemmProblem {
    const u32x4 *wq;        // packed codes
    const uint16_t *ws;     // packed scales
    const uint16_t *x;      // fp16 [M][K]
    float *out;             // fp32 [n_split][M][N]  (plain store)
    uint16_t *h;            // fp16 [M][N/2]        (SwiGLU epilogue)
    int M, N;               // tokens, valid packed rows
    int n_rb, n_chunks, n_groups;
    int n_split, gps;       // splits of the groups, groups per split
    int n_nb, n_mb, n_cols; // 128-row blocks, 128-token blocks, n_split * n_nb
    size_t split_stride;    // M * N
};

// Eight fp16 values q[k] (exact integers in [-8, 7]) from one code word:
// nibble i of the low half-word is element 2i, of the high half-word 2i+1.
// A nibble at bits 0-3 ORed into 0x6400 reads 1024 + u; at bits 4-7 ORed into
// 0x5400 it reads 64 + u (that exponent's unit is 1/16); u = q + 8.
__device__ __forceinline__ h8 dequant8(uint32_t w, uint32_t m_lo, uint32_t m_hi) {
    const uint32_t w8 = w >> 8;
    const h2 c_lo = {static_cast<_Float16>(-1032.0f), static_cast<_Float16>(-1032.0f)};
    const h2 c_hi = {static_cast<_Float16>(-72.0f), static_cast<_Float16>(-72.0f)};
    const h2 p0 = as_h2((w & m_lo) | 0x64006400u) + c_lo;
    const h2 p1 = as_h2((w & m_hi) | 0x54005400u) + c_hi;
    const h2 p2 = as_h2((w8 & m_lo) | 0x64006400u) + c_lo;
    const h2 p3 = as_h2((w8 & m_hi) | 0x54005400u) + c_hi;
    h8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// kSwiGLU: the rows are the W4_PERM_GATE_UP interleave (gate i, up i) and the
// launch has one split; the epilogue writes h[m][i] = fp16(silu(gate) * up)
// instead of the fp32 products.
template <bool kSwiGLU>
__global__ __launch_bounds__(kThreads) void w4_gemm_kernel(GemmProblem p) {
    __shared__ __attribute__((aligned(16))) uint16_t sx[2][kGemmBM * kGroup];
    // work-group -> (M block, split, 128-row block): the M blocks of one
    // weight column run back to back on one XCD (work-groups are dealt to the
    // 8 XCDs round-robin), so its codes are fetched from HBM about once.
    const int b = blockIdx.x;
    const int xcd = b & 7, j = b >> 3;
    const int mb = j % p.n_mb;
    const int col = (j / p.n_mb) * 8 + xcd;
    if (col >= p.n_cols) return;
    const int split = col / p.n_nb, nb = col - split * p.n_nb;
    const int g0 = split * p.gps;
    const int g1 = min(g0 + p.gps, p.n_groups);

    const int wave = wave_id();
    const int lane = threadIdx.x & 63;
    const int c32 = lane & 31, hf = lane >> 5;
    // wave -> 32 rows: half (wave & 1) of row block 2 nb + wave / 2
    const int rb = nb * 2 + (wave >> 1);
    const int rh = wave & 1;
    const bool wv = rb < p.n_rb;
    const int m0 = mb * kGemmBM;

    // activation staging: wave w fills rows 32 w .. 32 w + 31, four rows per
    // load instruction; lane -> row 32 w + 4 j + lane / 16, LDS chunk lane % 16
    // holding logical chunk (lane % 16) ^ (row % 16).  Rows past M repeat row
    // M - 1 (their products are never stored).
    const size_t ldx = static_cast<size_t>(p.n_groups) * kGroup;
    const int xrow0 = 32 * wave + (lane >> 4);
    auto load_x = [&](int g, int buf) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int row = xrow0 + 4 * jj;      // row % 16 = (xrow0 + 4 jj) % 16
            const int chunk = (lane & 15) ^ (row & 15);
            const uint16_t *src = p.x + static_cast<size_t>(min(m0 + row, p.M - 1)) * ldx + chunk * 8 + g * kGroup;
            __builtin_amdgcn_global_load_lds(src, &sx[buf][(32 * wave + 4 * jj) * kGroup], 16, 0, 0);
        }
    };
    // codes of the lane's row for the group: chunks 2 hf and 2 hf + 1
    u32x4 wreg[2];
    uint16_t sreg = 0;
    const u32x4 *wrow = p.wq + static_cast<size_t>(rb) * p.n_chunks * kRows + 32 * rh + c32;
    const uint16_t *srow = p.ws + static_cast<size_t>(rb) * p.n_groups * kRows + 32 * rh + c32;
    auto load_w = [&](int g) {
        if (!wv) return;
#pragma unroll
        for (int co = 0; co < 2; ++co) wreg[co] = wrow[static_cast<size_t>(4 * g + 2 * hf + co) * kRows];
        sreg = srow[static_cast<size_t>(g) * kRows];
    };

    double acc[4][16];      // [token sub-tile][C register]
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][i] = 0.0;

    const uint32_t m_lo = vreg_const(0x000F000Fu), m_hi = vreg_const(0x00F000F0u);
    load_x(g0, 0);
    load_w(g0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int g = g0; g < g1; ++g) {
        const int buf = (g - g0) & 1;
        const u32x4 wc0 = wreg[0], wc1 = wreg[1];
        const double sc = static_cast<double>(f16_to_f32(sreg));
        const bool more = g + 1 < g1;
        if (more) {
            load_x(g + 1, buf ^ 1);
            load_w(g + 1);
        }
        if (wv) {
            f32x16 t[4];
            // rows c32 + 32 ms share row % 16, hence one chunk swizzle
            const uint16_t *xa = &sx[buf][c32 * kGroup];
            const int sw = c32 & 15;
#pragma unroll
            for (int st = 0; st < 8; ++st) {
                const int ch = ((8 * hf + st) ^ sw) * 8;
                const uint32_t wword = st < 4 ? wc0[st] : wc1[st - 4];
                const h8 bq = dequant8(wword, m_lo, m_hi);
#pragma unroll
                for (int ms = 0; ms < 4; ++ms) {
                    const h8 a = *reinterpret_cast<const h8 *>(xa + 32 * ms * kGroup + ch);
                    if (st == 0) {
                        f32x16 z;
                        for (int i = 0; i < 16; ++i) z[i] = 0.0f;
                        t[ms] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bq, z, 0, 0, 0);
                    } else {
                        t[ms] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bq, t[ms], 0, 0, 0);
                    }
                }
            }
#pragma unroll
            for (int ms = 0; ms < 4; ++ms)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[ms][i] = fma(sc, static_cast<double>(t[ms][i]), acc[ms][i]);
        }
        // the next group's tile has landed in LDS (direct loads are counted
        // by vmcnt) before any wave passes the barrier
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    if (!wv) return;
    // C layout of a 32x32 tile: lane holds column c32 (a packed row) and the
    // 16 rows (tokens) 8 (i / 4) + 4 hf + i % 4.
    const int n = rb * kRows + 32 * rh + c32;
    if constexpr (kSwiGLU) {
        // gate (even column) and up (odd column) sit in neighbouring lanes
        const int half_n = p.N / 2;
#pragma unroll
        for (int ms = 0; ms < 4; ++ms)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const double g = acc[ms][i];
                const double u = shfl_xor1(g);
                const int m = m0 + 32 * ms + 8 * (i >> 2) + 4 * hf + (i & 3);
                if ((c32 & 1) == 0 && m < p.M && n < p.N)
                    p.h[static_cast<size_t>(m) * half_n + (n >> 1)] = f64_to_f16(g / (1.0 + exp(-g)) * u);
            }
        return;
    }
    if (n >= p.N) return;
    float *out = p.out + static_cast<size_t>(split) * p.split_stride;
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = m0 + 32 * ms + 8 * (i >> 2) + 4 * hf + (i & 3);
            if (m < p.M) out[static_cast<size_t>(m) * p.N + n] = static_cast<float>(acc[ms][i]);
        }
}

// y[m][n] = sum of the splits in order (fp64), stored as fp32.
__global__ __launch_bounds__(kThreads) void gemm_reduce_kernel(const float *part, int n_split, size_t stride,
                                                               size_t total, float *y) {
    for (size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x; i < total;
         i += static_cast<size_t>(gridDim.x) * kThreads) {
        double v = 0.0;
        for (int s = 0; s < n_split; ++s) v += static_cast<double>(part[s * stride + i]);
        y[i] = static_cast<float>(v);
    }
}

// ------------------------------------------------- per-token glue kernels --
// One work-group per token row m of the chunk (position pos0 + m).

__device__ __forceinline__ double block_sum4(double v, double *red) {
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return ((red[0] + red[1]) + red[2]) + red[3];
}

// a[m] = fp16(RMSNorm(x[m]) * w); x fp32 [d]
__device__ __forceinline__ void row_norm(const float *x, const uint16_t *w, uint16_t *a, int d, double eps,
                                         double *red) {
    double ss = 0.0;
    for (int i = threadIdx.x; i < d; i += kThreads) {
        const double v = x[i];
        ss += v * v;
    }
    ss = block_sum4(ss, red);
    const double r = sqrt(ss / d + eps);
    for (int i = threadIdx.x; i < d; i += kThreads)
        a[i] = f64_to_f16(static_cast<double>(x[i]) / r * static_cast<double>(f16_to_f32(w[i])));
}

// x[m] = embed[tokens[pos0 + m]] (fp32), a[m] = fp16(RMSNorm(x[m]) * ln1).
// Block 0 also appends the pages that start inside the chunk, clears the
// argmax key and sets the position to the chunk's last token.
__global__ __launch_bounds__(kThreads) void pf_embed_kernel(const uint16_t *embed, const int *tokens, int pos0,
                                                            int M, int d, const uint16_t *w, double eps,
                                                            float *x, uint16_t *a, int *page_table,
                                                            const int *free_list, StepState *st) {
    __shared__ double red[kThreads / 64];
    const int m = blockIdx.x;
    const int tok = tokens[pos0 + m];
    const uint16_t *row = embed + static_cast<size_t>(tok) * d;
    float *xr = x + static_cast<size_t>(m) * d;
    for (int i = threadIdx.x; i < d; i += kThreads) xr[i] = f16_to_f32(row[i]);
    __syncthreads();
    row_norm(xr, w, a + static_cast<size_t>(m) * d, d, eps, red);
    if (m == 0) {
        for (int lp = (pos0 + kPage - 1) / kPage + static_cast<int>(threadIdx.x); lp * kPage < pos0 + M;
             lp += kThreads)
            page_table[lp] = free_list[lp];
        if (threadIdx.x == 0) {
            st->best = 0ull;
            st->pos = pos0 + M - 1;
        }
    }
}

// QKV epilogue: y = sum of the GEMM splits + bias; RoPE on q and k; q to
// qbuf [M][n_qh][128], k and v into the layer's cache at the row's position.
// Packed row 2i of a head holds dim i and row 2i + 1 dim i + 64.
__global__ __launch_bounds__(kThreads) void pf_qkv_kernel(const float *part, int n_split, size_t stride, int N,
                                                          const uint16_t *bias, const double *rope, int pos0,
                                                          const int *page_table, uint16_t *qbuf, uint16_t *kc,
                                                          uint16_t *vc, int n_qh, int n_kvh) {
    const int m = blockIdx.x;
    const int pos = pos0 + m;
    const float *row = part + static_cast<size_t>(m) * N;
    const int phys = page_table[pos >> 4];
    for (int pr = threadIdx.x; pr < N / 2; pr += kThreads) {
        const int n = 2 * pr;
        double y0 = 0.0, y1 = 0.0;
        for (int s = 0; s < n_split; ++s) {
            const float2 v = *reinterpret_cast<const float2 *>(row + s * stride + n);
            y0 += static_cast<double>(v.x);
            y1 += static_cast<double>(v.y);
        }
        const int head = n >> 7;
        const int i = (n & 127) >> 1;
        y0 += static_cast<double>(f16_to_f32(bias[head * kHeadDim + i]));
        y1 += static_cast<double>(f16_to_f32(bias[head * kHeadDim + i + 64]));
        double o0 = y0, o1 = y1;
        if (head < n_qh + n_kvh) {
            const double c = rope[(static_cast<size_t>(pos) * 64 + i) * 2];
            const double sn = rope[(static_cast<size_t>(pos) * 64 + i) * 2 + 1];
            o0 = y0 * c - y1 * sn;
            o1 = y1 * c + y0 * sn;
        }
        const uint16_t h0 = f64_to_f16(o0), h1 = f64_to_f16(o1);
        if (head < n_qh) {
            uint16_t *q = qbuf + (static_cast<size_t>(m) * n_qh + head) * kHeadDim;
            q[i] = h0;
            q[i + 64] = h1;
        } else {
            const int kv = head - n_qh;
            const int jh = kv < n_kvh ? kv : kv - n_kvh;
            uint16_t *dst = (kv < n_kvh ? kc : vc) +
                            ((static_cast<size_t>(phys) * n_kvh + jh) * kPage + (pos & 15)) * kHeadDim;
            dst[i] = h0;
            dst[i + 64] = h1;
        }
    }
}

// x[m] += sum of the GEMM splits (fp64 sum in split order, stored fp32);
// a[m] = fp16(RMSNorm(x[m]) * w).  Four elements per thread step (d % 128 == 0).
__global__ __launch_bounds__(kThreads) void pf_resid_norm_kernel(const float *part, int n_split, size_t stride,
                                                                 int d, float *x, const uint16_t *w, double eps,
                                                                 uint16_t *a) {
    __shared__ double red[kThreads / 64];
    const int m = blockIdx.x;
    float4 *xr = reinterpret_cast<float4 *>(x + static_cast<size_t>(m) * d);
    const float4 *row = reinterpret_cast<const float4 *>(part + static_cast<size_t>(m) * d);
    const size_t st4 = stride / 4;
    const int d4 = d / 4;
    constexpr int kMaxV = 8;                       // d <= 8 * 4 * 256 (the model allows d <= 4096)
    float4 xv[kMaxV];
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < kMaxV; ++j) {
        const int i = threadIdx.x + j * kThreads;
        if (i < d4) {
            const float4 x0 = xr[i];
            double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
            for (int s = 0; s < n_split; ++s) {
                const float4 v = row[s * st4 + i];
                s0 += static_cast<double>(v.x);
                s1 += static_cast<double>(v.y);
                s2 += static_cast<double>(v.z);
                s3 += static_cast<double>(v.w);
            }
            float4 y;
            y.x = static_cast<float>(static_cast<double>(x0.x) + s0);
            y.y = static_cast<float>(static_cast<double>(x0.y) + s1);
            y.z = static_cast<float>(static_cast<double>(x0.z) + s2);
            y.w = static_cast<float>(static_cast<double>(x0.w) + s3);
            xr[i] = y;
            xv[j] = y;
            ss += static_cast<double>(y.x) * y.x + static_cast<double>(y.y) * y.y +
                  static_cast<double>(y.z) * y.z + static_cast<double>(y.w) * y.w;
        }
    }
    ss = block_sum4(ss, red);
    const double r = sqrt(ss / d + eps);
    const uint32_t *w2 = reinterpret_cast<const uint32_t *>(w);   // norm weights are 4-byte aligned
    uint2 *ar = reinterpret_cast<uint2 *>(a + static_cast<size_t>(m) * d);
#pragma unroll
    for (int j = 0; j < kMaxV; ++j) {
        const int i = threadIdx.x + j * kThreads;
        if (i < d4) {
            const uint2 wv = uint2{w2[2 * i], w2[2 * i + 1]};
            const float4 y = xv[j];
            const uint32_t h0 = f64_to_f16(static_cast<double>(y.x) / r * f16_to_f32(static_cast<uint16_t>(wv.x)));
            const uint32_t h1 = f64_to_f16(static_cast<double>(y.y) / r * f16_to_f32(static_cast<uint16_t>(wv.x >> 16)));
            const uint32_t h2v = f64_to_f16(static_cast<double>(y.z) / r * f16_to_f32(static_cast<uint16_t>(wv.y)));
            const uint32_t h3 = f64_to_f16(static_cast<double>(y.w) / r * f16_to_f32(static_cast<uint16_t>(wv.y >> 16)));
            ar[i] = uint2{h0 | (h1 << 16), h2v | (h3 << 16)};
        }
    }
}

// ------------------------------------------------ causal prefill attention --
//
// Query m of the chunk sits at position pos0 + m and attends to the cached
// positions 0..pos0 + m (the chunk's own K/V are already in the cache).
// Work-group = (query head, block of 32 queries); its 4 waves take every
// 4th block of 32 keys (2 pages) and merge their softmax states in wave
// order at the end.
// Per key block, on the matrix cores:
//   S^T (keys x queries) = K (keys x 128) . Q^T, 8 MFMA 32x32x16 steps;
//   the lane holding query c sees 16 of the block's keys, its partner lane
//   (c + 32) the other 16;
//   O^T (128 dims x queries) += V^T . P^T, 2 steps per 32 dims, with P^T
//   taken straight from the S^T registers (rounded to fp16) and V^T staged
//   through the wave's LDS slice.

struct PrefillAttnProblem {
    const uint16_t *q;          // fp16 [M][n_qh][128]
    const uint16_t *kpool, *vpool;
    const int *page_table;
    uint16_t *out;              // fp16 [M][n_qh][128]
    int M, n_qh, n_kvh, pos0, n_qb;
    float scale_log2;           // log2(e) / sqrt(128)
};

constexpr int kVtS = 40;                                // V^T row stride (halves): 32 keys + pad
constexpr int kAttnLdsBytes = 3 * 66 * 64 * 4;          // merge area (>= 4 waves x 128 x kVtS x 2)
static_assert(kAttnLdsBytes >= 4 * kHeadDim * kVtS * 2, "LDS too small for V^T slices");

__device__ __forceinline__ float xchg32(float v) {
    // value of the lane 32 apart
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(((threadIdx.x & 63) ^ 32) << 2,
                                                                  __builtin_bit_cast(int, v)));
}

__global__ __launch_bounds__(kThreads) void attn_prefill_kernel(PrefillAttnProblem p) {
    __shared__ __attribute__((aligned(16))) char lds[kAttnLdsBytes];
    const int wave = wave_id();
    const int lane = threadIdx.x & 63;
    const int c = lane & 31, hf = lane >> 5;
    // heavy query blocks first
    const int head = blockIdx.x % p.n_qh;
    const int qb = p.n_qb - 1 - static_cast<int>(blockIdx.x) / p.n_qh;
    const int kvh = head / (p.n_qh / p.n_kvh);
    const int m = qb * 32 + c;
    const int qpos = p.pos0 + m;
    const int kend = min(p.pos0 + qb * 32 + 32, p.pos0 + p.M);   // keys [0, kend) exist
    const int n_kb = (kend + 31) >> 5;

    // Q^T operand: query c, dims 64 hf + 8 t + e
    h8 qop[8];
    {
        const uint16_t *qr = p.q + (static_cast<size_t>(min(m, p.M - 1)) * p.n_qh + head) * kHeadDim + 64 * hf;
#pragma unroll
        for (int t = 0; t < 8; ++t) qop[t] = *reinterpret_cast<const h8 *>(qr + 8 * t);
    }
    uint16_t *vt = reinterpret_cast<uint16_t *>(lds) + wave * kHeadDim * kVtS;

    f32x16 o[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
        for (int i = 0; i < 16; ++i) o[s][i] = 0.0f;
    float mx = -INFINITY, l = 0.0f;

    for (int kb = wave; kb < n_kb; kb += 4) {
        // K operand: key c of the block, dims 64 hf + 8 t + e
        const int key = kb * 32 + c;
        h8 kop[8];
        if (key < kend) {
            const int phys = p.page_table[key >> 4];
            const uint16_t *kr = p.kpool + ((static_cast<size_t>(phys) * p.n_kvh + kvh) * kPage + (key & 15)) * kHeadDim +
                                 64 * hf;
#pragma unroll
            for (int t = 0; t < 8; ++t) kop[t] = *reinterpret_cast<const h8 *>(kr + 8 * t);
        } else {
#pragma unroll
            for (int t = 0; t < 8; ++t)
                for (int e = 0; e < 8; ++e) kop[t][e] = static_cast<_Float16>(0.0f);
        }
        // V rows: lane -> key pair (2 kp, 2 kp + 1), dims 32 qd .. 32 qd + 31
        const int kp = lane & 15, qd = lane >> 4;
        u32x4 va[4], vb[4];
        {
            const int k0 = kb * 32 + 2 * kp;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int kk = k0 + r;
                u32x4 *dst = r ? vb : va;
                if (kk < kend) {
                    const int phys = p.page_table[kk >> 4];
                    const u32x4 *vr = reinterpret_cast<const u32x4 *>(
                        p.vpool + ((static_cast<size_t>(phys) * p.n_kvh + kvh) * kPage + (kk & 15)) * kHeadDim + 32 * qd);
#pragma unroll
                    for (int t = 0; t < 4; ++t) dst[t] = vr[t];
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t) dst[t] = u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
        f32x16 s;
        for (int i = 0; i < 16; ++i) s[i] = 0.0f;
#pragma unroll
        for (int t = 0; t < 8; ++t) s = __builtin_amdgcn_mfma_f32_32x32x16_f16(kop[t], qop[t], s, 0, 0, 0);

        // V^T into the wave's LDS slice: row = dim, 2 keys per 32-bit word
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t a = va[t][w], bb = vb[t][w];
                const int dim = 32 * qd + 8 * t + 2 * w;
                *reinterpret_cast<uint32_t *>(vt + dim * kVtS + 2 * kp) = (a & 0xFFFFu) | (bb << 16);
                *reinterpret_cast<uint32_t *>(vt + (dim + 1) * kVtS + 2 * kp) = (a >> 16) | (bb & 0xFFFF0000u);
            }

        // scores of this lane: keys kb*32 + 8 (i/4) + 4 hf + i%4 for query c
        float bm = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int kk = kb * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
            const float v = kk <= qpos && kk < kend ? s[i] * p.scale_log2 : -INFINITY;
            s[i] = v;
            bm = fmaxf(bm, v);
        }
        bm = fmaxf(bm, xchg32(bm));
        const float mn = fmaxf(mx, bm);
        const float mu = mn == -INFINITY ? 0.0f : mn;
        const float alpha = __builtin_amdgcn_exp2f(mx - mu);
        mx = mn;
        h8 pb[2];
        float ps = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const _Float16 ph = static_cast<_Float16>(__builtin_amdgcn_exp2f(s[i] - mu));
            pb[i >> 3][i & 7] = ph;
            ps += static_cast<float>(ph);
        }
        l = l * alpha + ps;
#pragma unroll
        for (int sd = 0; sd < 4; ++sd)
            for (int i = 0; i < 16; ++i) o[sd][i] *= alpha;
        __builtin_amdgcn_s_waitcnt(0xc07f);   // this wave's LDS writes done (lgkmcnt 0)
        __builtin_amdgcn_wave_barrier();
        // O^T += V^T . P^T; V^T operand: dim 32 sd + c, keys 16 u + 4 hf + (0..3) and 16 u + 8 + 4 hf + (0..3)
#pragma unroll
        for (int sd = 0; sd < 4; ++sd) {
            const uint16_t *vr = vt + (32 * sd + c) * kVtS + 4 * hf;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const h4 lo = *reinterpret_cast<const h4 *>(vr + 16 * u);
                const h4 hi = *reinterpret_cast<const h4 *>(vr + 16 * u + 8);
                h8 vop;
                vop[0] = lo[0]; vop[1] = lo[1]; vop[2] = lo[2]; vop[3] = lo[3];
                vop[4] = hi[0]; vop[5] = hi[1]; vop[6] = hi[2]; vop[7] = hi[3];
                o[sd] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop, pb[u], o[sd], 0, 0, 0);
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
    l += xchg32(l);

    // merge the 4 waves in wave order; waves 1..3 park (m, l, o) in LDS
    __syncthreads();
    float *mg = reinterpret_cast<float *>(lds);
    if (wave > 0) {
        float *dst = mg + (wave - 1) * 66 * 64 + lane;
        dst[0] = mx;
        dst[64] = l;
#pragma unroll
        for (int sd = 0; sd < 4; ++sd)
            for (int i = 0; i < 16; ++i) dst[(2 + sd * 16 + i) * 64] = o[sd][i];
    }
    __syncthreads();
    if (wave != 0 || m >= p.M) return;
    float mall = mx;
    for (int w = 0; w < 3; ++w) mall = fmaxf(mall, mg[w * 66 * 64 + lane]);
    const float f0 = __builtin_amdgcn_exp2f(mx - mall);
    float lsum = l * f0;
#pragma unroll
    for (int sd = 0; sd < 4; ++sd)
        for (int i = 0; i < 16; ++i) o[sd][i] *= f0;
    for (int w = 0; w < 3; ++w) {
        const float *src = mg + w * 66 * 64 + lane;
        const float mw = src[0];
        const float fw = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - mall);
        lsum += src[64] * fw;
#pragma unroll
        for (int sd = 0; sd < 4; ++sd)
            for (int i = 0; i < 16; ++i) o[sd][i] += src[(2 + sd * 16 + i) * 64] * fw;
    }
    const float inv = 1.0f / lsum;
    uint16_t *dst = p.out + (static_cast<size_t>(m) * p.n_qh + head) * kHeadDim;
#pragma unroll
    for (int sd = 0; sd < 4; ++sd)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            h4 v;
            for (int e = 0; e < 4; ++e) v[e] = static_cast<_Float16>(o[sd][4 * g + e] * inv);
            *reinterpret_cast<h4 *>(dst + 32 * sd + 8 * g + 4 * hf) = v;
        }
}

}  // namespace w4

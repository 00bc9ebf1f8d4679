// gfx950 W4A16 batch-1 decode library: kernel entry points, glue kernels and
// the graph-captured decode step.  One translation unit holds every kernel so
// each template instantiation is registered exactly once.
#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <cmath>
#include <string>
#include <string.h>

#include <mutex>
#include <vector>

#include "w4_attn.hpp"
#include "w4_gemv.hpp"
#include "w4_gemv_stream.hpp"
#include "w4_persistent.hpp"
#include "w4_prefill.hpp"

namespace w4 {

// ------------------------------------------------------------ glue kernels --

// x = embed[tokens[pos]] as fp64, a = fp16(RMSNorm(x) * w) for the first
// layer; clears the argmax key.  One work-group.
__global__ __launch_bounds__(kThreads) void embed_kernel(const uint16_t *embed, const int *tokens,
                                                         StepState *st, double *x, const uint16_t *w,
                                                         uint16_t *a, int d, double eps) {
    __shared__ double red[kThreads / 64];
    const int tok = tokens[st->pos];
    const uint16_t *row = embed + static_cast<size_t>(tok) * d;
    double ss = 0.0;
    for (int i = threadIdx.x; i < d; i += kThreads) {
        const double v = static_cast<double>(f16_to_f32(row[i]));
        x[i] = v;
        ss += v * v;
    }
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const double r = sqrt((((red[0] + red[1]) + red[2]) + red[3]) / d + eps);
    for (int i = threadIdx.x; i < d; i += kThreads)
        a[i] = f64_to_f16(static_cast<double>(f16_to_f32(row[i])) / r * static_cast<double>(f16_to_f32(w[i])));
    if (threadIdx.x == 0) st->best = 0ull;
}

// Boundary-variant first node: the page of the position is appended.
__global__ void page_append_kernel(StepState *st, int *page_table, const int *free_list) {
    const int lp = st->pos >> 4;
    page_table[lp] = free_list[lp];
}

// Last node: greedy token, history update, position advance.
__global__ void finalize_kernel(StepState *st, int *tokens) {
    const int pos = st->pos;
    const unsigned long long key = st->best;
    const int tok = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key & 0xFFFFFFFFull));
    if (pos + 1 >= st->n_prompt) tokens[pos + 1] = tok;
    st->pos = pos + 1;
}

__global__ void reset_kernel(StepState *st, int n_prompt, unsigned *ctr, int n_ctr, int *err) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n_ctr; i += gridDim.x * blockDim.x) ctr[i] = 0u;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        st->pos = 0;
        st->n_prompt = n_prompt;
        st->best = 0ull;
        st->step = 0u;
        *err = 0;
    }
}

// -------------------------------------------------------------- launchers --

template <class Epi>
static hipError_t launch_w4(const W4Problem &p, const Epi &epi, hipStream_t s) {
    hipLaunchKernelGGL(w4_gemv_kernel<Epi>, dim3(p.n_rb * p.n_split), dim3(kThreads), 0, s, p, epi);
    return hipGetLastError();
}

static hipError_t launch_attn(int G, const AttnProblem &a, hipStream_t s) {
    const dim3 grid(a.n_kvh * a.n_split), block(kAttnThreads);
    switch (G) {
        case 1: hipLaunchKernelGGL(attn_decode_kernel<1>, grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL(attn_decode_kernel<2>, grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL(attn_decode_kernel<4>, grid, block, 0, s, a); break;
        case 7: hipLaunchKernelGGL(attn_decode_kernel<7>, grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL(attn_decode_kernel<8>, grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

static bool gqa_supported(int g) { return g == 1 || g == 2 || g == 4 || g == 7 || g == 8; }

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Workspace of split-K GEMVs that run one after another: a counter region
// of ctr_rb slots (the largest row-block count among them), then fp64
// partials.  A fixed counter region keeps every GEMV's counters away from any
// other GEMV's partials.
static size_t gemv_ws_bytes(int ctr_rb, size_t max_partials) {
    return align256(static_cast<size_t>(ctr_rb) * kGemvCtrStride * 4) + max_partials * 8;
}

static void gemv_ws_carve(void *ws, int ctr_rb, W4Problem &p) {
    p.counter = static_cast<unsigned *>(ws);
    p.partial = reinterpret_cast<double *>(static_cast<char *>(ws) +
                                           align256(static_cast<size_t>(ctr_rb) * kGemvCtrStride * 4));
}

static size_t gemv_partials(int n_rb, int n_split) {
    return n_split > 1 ? static_cast<size_t>(n_split) * n_rb * 64 : 0;
}

// The arrival counters sit in a region of fixed size at the start of the
// workspace, so partials of an earlier call with another shape never land on
// them; the last work-group of each kv head resets its counter, so a
// workspace that starts zero needs no clearing between calls.
constexpr int kAttnMaxKvh = 256;

static size_t attn_ws_bytes(int n_kvh, int G, int n_split) {
    return align256(static_cast<size_t>(kAttnMaxKvh) * kAttnCtrStride * 4) +
           align256(static_cast<size_t>(n_kvh) * n_split * G * 2 * 4) +
           static_cast<size_t>(n_kvh) * n_split * G * 128 * 4;
}

static void attn_ws_carve(void *ws, int n_kvh, int G, int n_split, AttnProblem &a) {
    char *b = static_cast<char *>(ws);
    a.counter = reinterpret_cast<unsigned *>(b);
    b += align256(static_cast<size_t>(kAttnMaxKvh) * kAttnCtrStride * 4);
    a.part_ml = reinterpret_cast<float *>(b);
    b += align256(static_cast<size_t>(n_kvh) * n_split * G * 2 * 4);
    a.part_acc = reinterpret_cast<float *>(b);
}

}  // namespace w4

using namespace w4;

// ============================================================ kernel calls ==

// Tiles of a standalone GEMV must fit an int (far beyond any matrix that fits
// in device memory: 2^31 tiles are 8 TiB of codes).
static bool sg_shape_ok(int64_t N, int64_t K) {
    return N >= 1 && K >= kGroup && K % kGroup == 0 && ((N + 63) / 64) * (K / kGroup) < (int64_t(1) << 31);
}

template <class Epi, bool kA8 = false, bool kShort = true>
static hipError_t launch_sg(const uint8_t *q, const uint16_t *sc, const void *x, int64_t N, int64_t K,
                            void *ws, const Epi &epi, hipStream_t s) {
    const int n_rb = static_cast<int>((N + 63) / 64), ng = static_cast<int>(K / kGroup);
    const SgGeom g = sg_geom(n_rb, ng);
    SgProblem p;
    p.wq = reinterpret_cast<const u32x4 *>(q);
    p.ws = sc;
    p.x = reinterpret_cast<const uint32_t *>(x);
    p.a8_scales = static_cast<uint32_t>(a8_scales_off(K));
    p.a8_sums = static_cast<uint32_t>(a8_sums_off(K));
    p.ng = ng;
    p.T = g.T;
    p.P = g.P;
    p.slot_stride = g.slot_stride;
    p.key_by_rb = g.key_by_rb;
    p.hdr = static_cast<unsigned *>(ws);
    p.ctr = reinterpret_cast<unsigned *>(static_cast<char *>(ws) + kSgHdrBytes);
    p.slots = reinterpret_cast<double *>(static_cast<char *>(ws) + kSgHdrBytes + sg_ctr_bytes(g));
    hipLaunchKernelGGL((sg_gemv_kernel<Epi, kA8, kShort>), dim3(g.P), dim3(kThreads), 0, s, p, epi);
    return hipGetLastError();
}

extern "C" size_t w4_gemv_ws_bytes(int64_t N, int64_t K) {
    if (N > (int64_t(1) << 31) - 64 || !sg_shape_ok(N, K)) return 0;
    return sg_ws_bytes(static_cast<int>((N + 63) / 64), static_cast<int>(K / kGroup));
}

extern "C" w4_status w4a16_gemv(const uint8_t *packed_q, const uint16_t *packed_s, const uint16_t *x,
                                uint16_t *y, int64_t N, int64_t K, void *workspace, size_t ws_bytes,
                                void *stream) {
    clear_error();
    W4_CHECK(N >= 1 && N <= (int64_t(1) << 31) - 64, W4_EINVAL, "bad N=%lld", (long long)N);
    W4_CHECK(K >= kGroup && K % kGroup == 0 && K <= (int64_t(1) << 24), W4_EINVAL,
             "K=%lld must be a positive multiple of 128", (long long)K);
    W4_CHECK(aligned16(packed_q) && aligned16(packed_s) && aligned16(x), W4_EALIGN,
             "packed_q, packed_s and x must be 16-byte aligned device pointers");
    W4_CHECK(y != nullptr && (reinterpret_cast<uintptr_t>(y) & 1) == 0, W4_EALIGN, "bad y pointer");
    W4_CHECK(sg_shape_ok(N, K), W4_EINVAL, "N=%lld x K=%lld is too large", (long long)N, (long long)K);
    const size_t need = w4_gemv_ws_bytes(N, K);
    W4_CHECK(ws_bytes >= need && aligned16(workspace), W4_EINVAL,
             "workspace of %zu bytes given (16-byte aligned), %zu needed", ws_bytes, need);
    W4_HIP(launch_sg(packed_q, packed_s, x, N, K, workspace, EpiStoreF16{y, static_cast<int>(N)},
                     static_cast<hipStream_t>(stream)));
    return W4_OK;
}

// ------------------------------------------- GEMV without allocation --
//
// For callers that cannot allocate: the workspace of w4a16_gemv lives in a
// fixed device array of this library.  In host code `scratch` names a
// host-side stand-in, not device memory, so its device address is looked up
// once per device and only that address is handed to kernels.

namespace {

constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (looked up on first use).
// The array is zero when the code object is loaded, and every w4a16_gemv
// launch leaves its workspace zero again, so it needs no clearing.
w4_status scratch_for_current_device(void **out) {
    int dev = -1;
    W4_HIP(hipGetDevice(&dev));
    W4_CHECK(dev >= 0 && dev < kMaxDevices, W4_EINVAL, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        W4_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
        W4_CHECK(ptr != nullptr && aligned16(ptr), W4_EHIP, "scratch symbol has no device address");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return W4_OK;
}

}  // namespace

extern "C" size_t w4_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

extern "C" w4_status w4a16_gemv_noalloc(const uint8_t *packed_q, const uint16_t *packed_s, const uint16_t *x,
                                        uint16_t *y, int64_t N, int64_t K, void *stream) {
    clear_error();
    W4_CHECK(N >= 1 && N <= (int64_t(1) << 31) - 64, W4_EINVAL, "bad N=%lld", (long long)N);
    W4_CHECK(K >= kGroup && K % kGroup == 0 && K <= (int64_t(1) << 24), W4_EINVAL,
             "K=%lld must be a positive multiple of 128", (long long)K);
    W4_CHECK(sg_shape_ok(N, K), W4_EINVAL, "N=%lld x K=%lld is too large", (long long)N, (long long)K);
    const size_t need = w4_gemv_ws_bytes(N, K);
    W4_CHECK(need > 0 && need <= kNoAllocScratchBytes, W4_EINVAL,
             "N=%lld x K=%lld needs %zu bytes of workspace, beyond the fixed %zu", (long long)N, (long long)K, need,
             kNoAllocScratchBytes);
    void *ws = nullptr;
    const w4_status st = scratch_for_current_device(&ws);
    if (st != W4_OK) return st;
    return w4a16_gemv(packed_q, packed_s, x, y, N, K, ws, kNoAllocScratchBytes, stream);
}

// ----------------------------------------------------- int8 activations --

extern "C" size_t w4a8_act_bytes(int64_t K) {
    if (K < kGroup || K % kGroup || K > (int64_t(1) << 24)) return 0;
    return a8_act_bytes(K);
}

extern "C" w4_status w4a8_quantize_act(const uint16_t *x, int64_t K, void *act, void *stream) {
    clear_error();
    W4_CHECK(K >= kGroup && K % kGroup == 0 && K <= (int64_t(1) << 24), W4_EINVAL,
             "K=%lld must be a positive multiple of 128", (long long)K);
    W4_CHECK(aligned16(x) && aligned16(act), W4_EALIGN, "x and act must be 16-byte aligned device pointers");
    char *a = static_cast<char *>(act);
    hipLaunchKernelGGL(a8_quantize_kernel, dim3(static_cast<unsigned>(K / kGroup)), dim3(64), 0,
                       static_cast<hipStream_t>(stream), x, reinterpret_cast<int8_t *>(a),
                       reinterpret_cast<float *>(a + a8_scales_off(K)), reinterpret_cast<int *>(a + a8_sums_off(K)));
    W4_HIP(hipGetLastError());
    return W4_OK;
}

extern "C" w4_status w4a8_gemv(const uint8_t *packed_q, const uint16_t *packed_s, const void *act, uint16_t *y,
                               int64_t N, int64_t K, void *workspace, size_t ws_bytes, void *stream) {
    clear_error();
    W4_CHECK(N >= 1 && N <= (int64_t(1) << 31) - 64, W4_EINVAL, "bad N=%lld", (long long)N);
    W4_CHECK(K >= kGroup && K % kGroup == 0 && K <= (int64_t(1) << 24), W4_EINVAL,
             "K=%lld must be a positive multiple of 128", (long long)K);
    W4_CHECK(aligned16(packed_q) && aligned16(packed_s) && aligned16(act), W4_EALIGN,
             "packed_q, packed_s and act must be 16-byte aligned device pointers");
    W4_CHECK(y != nullptr && (reinterpret_cast<uintptr_t>(y) & 1) == 0, W4_EALIGN, "bad y pointer");
    W4_CHECK(sg_shape_ok(N, K), W4_EINVAL, "N=%lld x K=%lld is too large", (long long)N, (long long)K);
    const size_t need = w4_gemv_ws_bytes(N, K);
    W4_CHECK(ws_bytes >= need && aligned16(workspace), W4_EINVAL,
             "workspace of %zu bytes given (16-byte aligned), %zu needed", ws_bytes, need);
    W4_HIP((launch_sg<EpiStoreF16, true>(packed_q, packed_s, act, N, K, workspace, EpiStoreF16{y, static_cast<int>(N)},
                                         static_cast<hipStream_t>(stream))));
    return W4_OK;
}

extern "C" size_t w4_mlp_ws_bytes(int64_t D, int64_t F) {
    if (D < kGroup || D % kGroup || F < kGroup || F % kGroup || D > (1 << 24) || F > (1 << 24)) return 0;
    if (!sg_shape_ok(2 * F, D) || !sg_shape_ok(D, F)) return 0;
    return std::max(w4_gemv_ws_bytes(2 * F, D), w4_gemv_ws_bytes(D, F));
}

extern "C" w4_status w4a16_mlp(const uint8_t *gu_q, const uint16_t *gu_s, const uint8_t *down_q,
                               const uint16_t *down_s, const uint16_t *x, uint16_t *h, uint16_t *y, int64_t D,
                               int64_t F, void *workspace, size_t ws_bytes, void *stream) {
    clear_error();
    W4_CHECK(D >= kGroup && D % kGroup == 0 && F >= kGroup && F % kGroup == 0 && D <= (1 << 24) && F <= (1 << 24),
             W4_EINVAL, "D=%lld and F=%lld must be positive multiples of 128", (long long)D, (long long)F);
    W4_CHECK(aligned16(gu_q) && aligned16(gu_s) && aligned16(down_q) && aligned16(down_s) && aligned16(x) &&
                 aligned16(h) && aligned16(workspace) && y != nullptr,
             W4_EALIGN, "weights, x, h and workspace must be 16-byte aligned device pointers");
    W4_CHECK(sg_shape_ok(2 * F, D) && sg_shape_ok(D, F), W4_EINVAL, "D=%lld, F=%lld too large", (long long)D,
             (long long)F);
    const size_t need = w4_mlp_ws_bytes(D, F);
    W4_CHECK(ws_bytes >= need, W4_EINVAL, "workspace of %zu bytes given, %zu needed", ws_bytes, need);
    hipStream_t s = static_cast<hipStream_t>(stream);
    W4_HIP((launch_sg<EpiSwiGLU, false, false>(gu_q, gu_s, x, 2 * F, D, workspace, EpiSwiGLU{h, static_cast<int>(F)},
                                              s)));
    W4_HIP(launch_sg(down_q, down_s, h, D, F, workspace, EpiStoreF16{y, static_cast<int>(D)}, s));
    return W4_OK;
}

extern "C" size_t w4_attn_ws_bytes(int32_t n_qh, int32_t n_kvh, int32_t n_pages_max) {
    if (n_kvh < 1 || n_kvh > kAttnMaxKvh || n_qh < 1 || n_qh % n_kvh || n_pages_max < 1) return 0;
    return attn_ws_bytes(n_kvh, n_qh / n_kvh, attn_n_split(n_pages_max));
}

extern "C" w4_status paged_attn_decode(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                                       const int32_t *page_table, int32_t ctx_len, int32_t n_qh,
                                       int32_t n_kvh, int32_t head_dim, int32_t n_pages_max, float scale,
                                       uint16_t *out, void *workspace, size_t ws_bytes, void *stream) {
    clear_error();
    W4_CHECK(head_dim == kHeadDim, W4_EINVAL, "head_dim must be 128 (got %d)", head_dim);
    W4_CHECK(n_kvh >= 1 && n_kvh <= kAttnMaxKvh && n_qh >= 1 && n_qh % n_kvh == 0 && gqa_supported(n_qh / n_kvh),
             W4_EINVAL,
             "n_qh=%d / n_kvh=%d must be one of 1, 2, 4, 7, 8", n_qh, n_kvh);
    W4_CHECK(n_pages_max >= 1 && ctx_len >= 1 && static_cast<int64_t>(ctx_len) <= int64_t(kPage) * n_pages_max,
             W4_EINVAL, "ctx_len=%d outside [1, 16*n_pages_max=%lld]", ctx_len,
             (long long)(int64_t(kPage) * n_pages_max));
    W4_CHECK(std::isfinite(scale), W4_EINVAL, "scale must be finite");
    W4_CHECK(aligned16(q) && aligned16(k_pool) && aligned16(v_pool) && aligned16(out) && aligned16(workspace) &&
                 page_table != nullptr,
             W4_EALIGN, "q, pools, out and workspace must be 16-byte aligned device pointers");
    const int G = n_qh / n_kvh;
    const int n_split = attn_n_split(n_pages_max);
    const size_t need = attn_ws_bytes(n_kvh, G, n_split);
    W4_CHECK(ws_bytes >= need, W4_EINVAL, "workspace of %zu bytes given, %zu needed", ws_bytes, need);
    AttnProblem a;
    a.q = q;
    a.kpool = k_pool;
    a.vpool = v_pool;
    a.page_table = page_table;
    a.pos_ptr = nullptr;
    a.ctx = ctx_len;
    a.n_kvh = n_kvh;
    a.pages_per_split = attn_pages_per_split(n_pages_max);
    a.n_split = n_split;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.out = out;
    attn_ws_carve(workspace, n_kvh, G, n_split, a);
    W4_HIP(launch_attn(G, a, static_cast<hipStream_t>(stream)));
    return W4_OK;
}

// ------------------------------------------------------------ W4A16 GEMM --

namespace w4 {

constexpr int kGemmTarget = 512;   // work-groups a GEMM launch aims for (2 per CU)

struct GemmGeom {
    int n_rb, n_nb, n_mb, n_groups, n_split, gps, n_cols, grid;
};

// Launch geometry of w4_gemm_kernel: 128-token x 128-row tiles, the groups
// split (at most max_split ways) as far as the launch still fits in one round
// of kGemmTarget resident work-groups, the grid padded to a multiple of 8
// columns for the XCD mapping.  A grid just past one round runs its last
// work-groups as a second, nearly empty round (measured on the 7B shapes at
// 512 tokens: down 112 -> 91 us, QKV 36 -> 31 us, O 32 -> 25 us when the
// splits drop from 5, 4, 5 to 4, 3, 4).
static GemmGeom gemm_geom(int M, int N, int K, int max_split = 8) {
    GemmGeom g;
    g.n_rb = (N + kRows - 1) / kRows;
    g.n_nb = (g.n_rb + 1) / 2;
    g.n_mb = (M + kGemmBM - 1) / kGemmBM;
    g.n_groups = K / kGroup;
    const int s_max = std::max(1, std::min(max_split, g.n_groups));
    for (int s = s_max; s >= 1; --s) {
        g.gps = (g.n_groups + s - 1) / s;
        g.n_split = (g.n_groups + g.gps - 1) / g.gps;
        g.n_cols = g.n_split * g.n_nb;
        g.grid = g.n_mb * ((g.n_cols + 7) / 8) * 8;
        if (g.grid <= kGemmTarget) break;
    }
    return g;
}

// out != nullptr: fp32 split partials; otherwise (one split) the SwiGLU
// epilogue writes fp16 h [M][N/2].
static hipError_t launch_gemm(const GemmGeom &g, const uint8_t *q, const uint16_t *s, const uint16_t *x, int M,
                              int N, float *out, hipStream_t st, uint16_t *h = nullptr) {
    GemmProblem p;
    p.wq = reinterpret_cast<const u32x4 *>(q);
    p.ws = s;
    p.x = x;
    p.out = out;
    p.h = h;
    p.M = M;
    p.N = N;
    p.n_rb = g.n_rb;
    p.n_chunks = g.n_groups * (kGroup / kChunk);
    p.n_groups = g.n_groups;
    p.n_split = g.n_split;
    p.gps = g.gps;
    p.n_nb = g.n_nb;
    p.n_mb = g.n_mb;
    p.n_cols = g.n_cols;
    p.split_stride = static_cast<size_t>(M) * N;
    if (out != nullptr) {
        hipLaunchKernelGGL(w4_gemm_kernel<false>, dim3(g.grid), dim3(kThreads), 0, st, p);
    } else {
        if (g.n_split != 1 || h == nullptr || N % 2) return hipErrorInvalidValue;
        hipLaunchKernelGGL(w4_gemm_kernel<true>, dim3(g.grid), dim3(kThreads), 0, st, p);
    }
    return hipGetLastError();
}

// Largest split-K partial area (floats) of an M x N x K GEMM over every M in [1, m_max].
static size_t gemm_part_floats_max(int m_max, int N, int K) {
    size_t best = 0;
    for (int mb = 1; mb * kGemmBM - (kGemmBM - 1) <= m_max; ++mb) {
        const int M = std::min(mb * kGemmBM, m_max);
        const GemmGeom g = gemm_geom(M, N, K);
        best = std::max(best, static_cast<size_t>(g.n_split) * M * N);
    }
    return best;
}

static hipError_t launch_attn_prefill(const uint16_t *q, const uint16_t *kc, const uint16_t *vc, const int *pt,
                                      uint16_t *out, int M, int n_qh, int n_kvh, int pos0, float scale,
                                      hipStream_t st) {
    PrefillAttnProblem a;
    a.q = q;
    a.kpool = kc;
    a.vpool = vc;
    a.page_table = pt;
    a.out = out;
    a.M = M;
    a.n_qh = n_qh;
    a.n_kvh = n_kvh;
    a.pos0 = pos0;
    a.n_qb = (M + 31) / 32;
    a.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
    hipLaunchKernelGGL(attn_prefill_kernel, dim3(n_qh * a.n_qb), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace w4

extern "C" size_t w4_gemm_ws_bytes(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || M > (1 << 20) || N < 1 || N > (int64_t(1) << 30) || K < kGroup || K % kGroup ||
        K > (int64_t(1) << 24))
        return 0;
    const GemmGeom g = gemm_geom(static_cast<int>(M), static_cast<int>(N), static_cast<int>(K));
    return g.n_split > 1 ? static_cast<size_t>(g.n_split) * M * N * sizeof(float) : 16;
}

extern "C" w4_status w4a16_gemm(const uint8_t *packed_q, const uint16_t *packed_s, const uint16_t *x, float *y,
                                int64_t M, int64_t N, int64_t K, void *workspace, size_t ws_bytes, void *stream) {
    clear_error();
    W4_CHECK(M >= 1 && M <= (1 << 20), W4_EINVAL, "bad M=%lld", (long long)M);
    W4_CHECK(N >= 1 && N <= (int64_t(1) << 30) && M * N <= (int64_t(1) << 34), W4_EINVAL, "bad N=%lld",
             (long long)N);
    W4_CHECK(K >= kGroup && K % kGroup == 0 && K <= (int64_t(1) << 24), W4_EINVAL,
             "K=%lld must be a positive multiple of 128", (long long)K);
    W4_CHECK(aligned16(packed_q) && aligned16(packed_s) && aligned16(x), W4_EALIGN,
             "packed_q, packed_s and x must be 16-byte aligned device pointers");
    W4_CHECK(y != nullptr && (reinterpret_cast<uintptr_t>(y) & 3) == 0, W4_EALIGN, "bad y pointer");
    const GemmGeom g = gemm_geom(static_cast<int>(M), static_cast<int>(N), static_cast<int>(K));
    const size_t need = w4_gemm_ws_bytes(M, N, K);
    W4_CHECK(ws_bytes >= need && aligned16(workspace), W4_EINVAL,
             "workspace of %zu bytes given (16-byte aligned), %zu needed", ws_bytes, need);
    hipStream_t s = static_cast<hipStream_t>(stream);
    float *dst = g.n_split > 1 ? static_cast<float *>(workspace) : y;
    W4_HIP(launch_gemm(g, packed_q, packed_s, x, static_cast<int>(M), static_cast<int>(N), dst, s));
    if (g.n_split > 1) {
        const size_t total = static_cast<size_t>(M) * N;
        const int blocks = static_cast<int>(std::min<size_t>((total + kThreads - 1) / kThreads, 4096));
        hipLaunchKernelGGL(gemm_reduce_kernel, dim3(blocks), dim3(kThreads), 0, s, dst, g.n_split, total, total, y);
        W4_HIP(hipGetLastError());
    }
    return W4_OK;
}

extern "C" w4_status paged_attn_prefill(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                                        const int32_t *page_table, int32_t pos0, int32_t n_tokens, int32_t n_qh,
                                        int32_t n_kvh, int32_t head_dim, float scale, uint16_t *out,
                                        void *stream) {
    clear_error();
    W4_CHECK(head_dim == kHeadDim, W4_EINVAL, "head_dim must be 128");
    W4_CHECK(n_kvh >= 1 && n_qh >= n_kvh && n_qh % n_kvh == 0 && n_qh <= 1024, W4_EINVAL,
             "n_qh=%d must be a multiple of n_kvh=%d", n_qh, n_kvh);
    W4_CHECK(n_tokens >= 1 && n_tokens <= (1 << 20) && pos0 >= 0 && pos0 <= (1 << 24), W4_EINVAL,
             "bad pos0=%d n_tokens=%d", pos0, n_tokens);
    W4_CHECK(std::isfinite(scale) && scale > 0.0f, W4_EINVAL, "scale must be positive");
    W4_CHECK(aligned16(q) && aligned16(k_pool) && aligned16(v_pool) && aligned16(out) && page_table != nullptr,
             W4_EALIGN, "q, pools and out must be 16-byte aligned device pointers");
    W4_HIP(launch_attn_prefill(q, k_pool, v_pool, page_table, out, n_tokens, n_qh, n_kvh, pos0, scale,
                               static_cast<hipStream_t>(stream)));
    return W4_OK;
}

// ================================================================== model ==

struct w4_model {
    w4_model_config cfg;
    std::vector<const uint8_t *> qkv_q, o_q, gu_q, down_q;
    std::vector<const uint16_t *> qkv_s, qkv_bias, o_s, gu_s, down_s, ln1, ln2;
    const uint16_t *embed, *lnf, *lm_head;
    uint16_t *k_cache, *v_cache;
    int32_t *page_table, *tokens;
    const int32_t *free_list;
    float *logits;

    // library-owned device memory (one allocation, carved)
    void *arena;
    void *pk_arena;
    StepState *state;
    double *x;          // residual [d]
    uint16_t *a;        // normed input [d]
    uint16_t *qbuf;     // q after RoPE [n_qh*128]
    uint16_t *o;        // attention output [n_qh*128]
    uint16_t *h;        // SwiGLU output [d_ff]
    double *rope;       // [max_pos][64][2]
    void *gemv_ws;      // shared by the GEMVs of a step (stream-ordered)
    double *norm_ss;    // per-row-block sums of squares of the fused RMSNorm
    unsigned *norm_ctr; // row-block arrivals of the fused RMSNorm
    void *attn_ws;
    size_t gemv_ws_size;

    // per-GEMV launch geometry
    int rb_qkv, sp_qkv, rb_o, sp_o, rb_gu, sp_gu, rb_down, sp_down, rb_head;
    int ctr_rb;               // counter slots at the start of gemv_ws
    int attn_pps, attn_split;

    // persistent step
    PKParams pk;
    PKLayer *pk_layers;       // device array
    PKParams *pk_dev;         // device copy of pk
    size_t trace_bytes = 0;   // phase-timestamp buffer (trace builds)
    size_t resid_stride = 0;  // floats between the residual-stream vectors
    int pk_grid;              // resident work-groups
    int n_ctr;

    // prefill scratch (kPrefillMax token rows)
    void *pf_arena;
    float *pf_x;        // residual [rows][d]
    uint16_t *pf_a;     // normed input [rows][d]
    uint16_t *pf_q;     // q after RoPE [rows][n_qh*128]
    uint16_t *pf_o;     // attention output [rows][n_qh*128]
    uint16_t *pf_h;     // SwiGLU output [rows][d_ff]
    float *pf_part;     // GEMM split-K partials
    size_t pf_part_floats;

    hipStream_t cap_stream;
    hipGraphExec_t exec[2];   // persistent step: [0] no page boundary, [1] page boundary
    hipGraphExec_t exec_multi[2];   // kernel-per-op step, same variants
    hipGraphExec_t exec_a8[2];      // persistent int8-activation step (captured on first use)
    bool a8_ok;                     // the int8 variant's staged groups fit its registers
    int pos;                  // host mirror of the device position
    int n_prompt;
    int launches;
};

namespace w4 {

static size_t layer_kv_elems(const w4_model *m) {
    return static_cast<size_t>(m->cfg.max_pages) * m->cfg.n_kv_heads * kPage * kHeadDim;
}

static W4Problem w4_problem(const w4_model *m, const uint8_t *q, const uint16_t *s, const uint16_t *x,
                            int n_rb, int n_split, int K) {
    W4Problem p;
    p.wq = reinterpret_cast<const u32x4 *>(q);
    p.ws = s;
    p.x = reinterpret_cast<const uint32_t *>(x);
    p.n_groups = K / kGroup;
    p.n_rb = n_rb;
    p.n_split = n_split;
    gemv_ws_carve(m->gemv_ws, m->ctr_rb, p);
    return p;
}

// Enqueues one whole decode step (boundary: with the page append first).
static hipError_t enqueue_step(w4_model *m, bool boundary, hipStream_t s) {
    const w4_model_config &c = m->cfg;
    const int d = c.d_model, f = c.d_ff, qd = c.n_q_heads * kHeadDim;
    const int G = c.n_q_heads / c.n_kv_heads;
    const int *pos_ptr = &m->state->pos;
    int launches = 0;
    hipError_t e;
#define W4_Q(call)                          \
    do {                                    \
        e = (call);                         \
        if (e != hipSuccess) return e;      \
        ++launches;                         \
    } while (0)
    if (boundary) {
        hipLaunchKernelGGL(page_append_kernel, dim3(1), dim3(1), 0, s, m->state, m->page_table, m->free_list);
        W4_Q(hipGetLastError());
    }
    hipLaunchKernelGGL(embed_kernel, dim3(1), dim3(kThreads), 0, s, m->embed, m->tokens, m->state, m->x, m->ln1[0],
                       m->a, d, double(c.eps));
    W4_Q(hipGetLastError());
    for (int l = 0; l < c.n_layers; ++l) {
        uint16_t *kc = m->k_cache + l * layer_kv_elems(m);
        uint16_t *vc = m->v_cache + l * layer_kv_elems(m);
        // a holds RMSNorm(x) * ln1[l] (from the embedding or the previous down GEMV)
        EpiQKV eq{m->qkv_bias[l], m->rope, pos_ptr, m->page_table, m->qbuf, kc, vc, c.n_q_heads, c.n_kv_heads};
        W4_Q(launch_w4(w4_problem(m, m->qkv_q[l], m->qkv_s[l], m->a, m->rb_qkv, m->sp_qkv, d), eq, s));
        AttnProblem a;
        a.q = m->qbuf;
        a.kpool = kc;
        a.vpool = vc;
        a.page_table = m->page_table;
        a.pos_ptr = pos_ptr;
        a.ctx = 0;
        a.n_kvh = c.n_kv_heads;
        a.pages_per_split = m->attn_pps;
        a.n_split = m->attn_split;
        a.scale_log2 = static_cast<float>(1.4426950408889634 / sqrt(double(kHeadDim)));
        a.out = m->o;
        attn_ws_carve(m->attn_ws, c.n_kv_heads, G, m->attn_split, a);
        W4_Q(launch_attn(G, a, s));
        // x += Wo o, then a = RMSNorm(x) * ln2[l]
        EpiResidualNorm eo{m->x, d, m->ln2[l], m->a, m->norm_ss, m->norm_ctr, double(c.eps)};
        W4_Q(launch_w4(w4_problem(m, m->o_q[l], m->o_s[l], m->o, m->rb_o, m->sp_o, qd), eo, s));
        W4_Q(launch_w4(w4_problem(m, m->gu_q[l], m->gu_s[l], m->a, m->rb_gu, m->sp_gu, d), EpiSwiGLU{m->h, f}, s));
        // x += Wd h, then a = RMSNorm(x) * (ln1[l+1] or the final norm)
        const uint16_t *next_w = l + 1 < c.n_layers ? m->ln1[l + 1] : m->lnf;
        EpiResidualNorm ed{m->x, d, next_w, m->a, m->norm_ss, m->norm_ctr, double(c.eps)};
        W4_Q(launch_w4(w4_problem(m, m->down_q[l], m->down_s[l], m->h, m->rb_down, m->sp_down, f), ed, s));
    }
    F16Problem hp;
    hp.w = reinterpret_cast<const u32x4 *>(m->lm_head);
    hp.x = reinterpret_cast<const uint32_t *>(m->a);
    hp.n_chunks = d / 8;
    hp.n_rb = m->rb_head;
    hp.n = c.vocab;
    hp.out = m->logits;
    hp.best = &m->state->best;
    hipLaunchKernelGGL(f16_gemv_kernel, dim3(m->rb_head), dim3(kThreads), 0, s, hp);
    W4_Q(hipGetLastError());
    hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(1), 0, s, m->state, m->tokens);
    W4_Q(hipGetLastError());
#undef W4_Q
    m->launches = launches - (boundary ? 1 : 0);
    return hipSuccess;
}

static hipError_t enqueue_persistent(w4_model *m, bool boundary, hipStream_t s, bool a8 = false) {
    if (boundary) {
        hipLaunchKernelGGL(page_append_kernel, dim3(1), dim3(1), 0, s, m->state, m->page_table, m->free_list);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a8)
        hipLaunchKernelGGL(decode_persistent_kernel<true>, dim3(m->pk_grid), dim3(kPkThreads), 0, s,
                           static_cast<const PKParams *>(m->pk_dev));
    else
        hipLaunchKernelGGL(decode_persistent_kernel<false>, dim3(m->pk_grid), dim3(kPkThreads), 0, s,
                           static_cast<const PKParams *>(m->pk_dev));
    return hipGetLastError();
}

static w4_status capture(w4_model *m, bool boundary, bool multi, hipGraphExec_t *out, bool a8 = false) {
    hipGraph_t g = nullptr;
    W4_HIP(hipStreamBeginCapture(m->cap_stream, hipStreamCaptureModeThreadLocal));
    hipError_t e = multi ? enqueue_step(m, boundary, m->cap_stream) : enqueue_persistent(m, boundary, m->cap_stream, a8);
    hipError_t e2 = hipStreamEndCapture(m->cap_stream, &g);
    if (e != hipSuccess || e2 != hipSuccess) {
        if (g) (void)hipGraphDestroy(g);
        return fail(W4_EHIP, "step capture failed: %s", hipGetErrorString(e != hipSuccess ? e : e2));
    }
    e = hipGraphInstantiate(out, g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    W4_HIP(e);
    return W4_OK;
}

static void model_free(w4_model *m) {
    if (!m) return;
    for (int i = 0; i < 2; ++i) {
        if (m->exec[i]) (void)hipGraphExecDestroy(m->exec[i]);
        if (m->exec_multi[i]) (void)hipGraphExecDestroy(m->exec_multi[i]);
        if (m->exec_a8[i]) (void)hipGraphExecDestroy(m->exec_a8[i]);
    }
    if (m->cap_stream) (void)hipStreamDestroy(m->cap_stream);
    if (m->arena) (void)hipFree(m->arena);
    if (m->pk_arena) (void)hipFree(m->pk_arena);
    if (m->pf_arena) (void)hipFree(m->pf_arena);
    delete m;
}

// Prefill scratch for kPrefillMax token rows.
static w4_status setup_prefill(w4_model *m) {
    const w4_model_config &c = m->cfg;
    const int d = c.d_model, f = c.d_ff, qd = c.n_q_heads * kHeadDim;
    const int qkv_rows = (c.n_q_heads + 2 * c.n_kv_heads) * kHeadDim;
    const size_t R = kPrefillMax;
    size_t part = gemm_part_floats_max(kPrefillMax, qkv_rows, d);
    part = std::max(part, gemm_part_floats_max(kPrefillMax, d, qd));
    part = std::max(part, gemm_part_floats_max(kPrefillMax, d, f));
    const size_t sizes[6] = {align256(R * d * 4), align256(R * d * 2), align256(R * qd * 2),
                             align256(R * qd * 2), align256(R * f * 2), align256(part * 4)};
    size_t total = 0;
    for (size_t s : sizes) total += s;
    W4_HIP(hipMalloc(&m->pf_arena, total));
    char *b = static_cast<char *>(m->pf_arena);
    m->pf_x = reinterpret_cast<float *>(b); b += sizes[0];
    m->pf_a = reinterpret_cast<uint16_t *>(b); b += sizes[1];
    m->pf_q = reinterpret_cast<uint16_t *>(b); b += sizes[2];
    m->pf_o = reinterpret_cast<uint16_t *>(b); b += sizes[3];
    m->pf_h = reinterpret_cast<uint16_t *>(b); b += sizes[4];
    m->pf_part = reinterpret_cast<float *>(b);
    m->pf_part_floats = part;
    return W4_OK;
}

// Enqueues the prefill of tokens [pos0, pos0 + M): every layer over the M
// rows, then the lm_head on the last row and the greedy token.
static hipError_t enqueue_prefill(w4_model *m, int pos0, int M, hipStream_t s) {
    const w4_model_config &c = m->cfg;
    const int d = c.d_model, f = c.d_ff, qd = c.n_q_heads * kHeadDim;
    const int qkv_rows = (c.n_q_heads + 2 * c.n_kv_heads) * kHeadDim;
    const double eps = c.eps;
    const float scale = static_cast<float>(1.0 / sqrt(double(kHeadDim)));
    hipError_t e;
#define W4_PF(call)                     \
    do {                                \
        call;                           \
        e = hipGetLastError();          \
        if (e != hipSuccess) return e;  \
    } while (0)
    W4_PF(hipLaunchKernelGGL(pf_embed_kernel, dim3(M), dim3(kThreads), 0, s, m->embed, m->tokens, pos0, M, d,
                             m->ln1[0], eps, m->pf_x, m->pf_a, m->page_table, m->free_list, m->state));
    const GemmGeom g_qkv = gemm_geom(M, qkv_rows, d), g_o = gemm_geom(M, d, qd), g_gu = gemm_geom(M, 2 * f, d, 1),
                   g_dn = gemm_geom(M, d, f);
    for (int l = 0; l < c.n_layers; ++l) {
        uint16_t *kc = m->k_cache + l * layer_kv_elems(m);
        uint16_t *vc = m->v_cache + l * layer_kv_elems(m);
        e = launch_gemm(g_qkv, m->qkv_q[l], m->qkv_s[l], m->pf_a, M, qkv_rows, m->pf_part, s);
        if (e != hipSuccess) return e;
        W4_PF(hipLaunchKernelGGL(pf_qkv_kernel, dim3(M), dim3(kThreads), 0, s, m->pf_part, g_qkv.n_split,
                                 static_cast<size_t>(M) * qkv_rows, qkv_rows, m->qkv_bias[l], m->rope, pos0,
                                 m->page_table, m->pf_q, kc, vc, c.n_q_heads, c.n_kv_heads));
        e = launch_attn_prefill(m->pf_q, kc, vc, m->page_table, m->pf_o, M, c.n_q_heads, c.n_kv_heads, pos0, scale, s);
        if (e != hipSuccess) return e;
        e = launch_gemm(g_o, m->o_q[l], m->o_s[l], m->pf_o, M, d, m->pf_part, s);
        if (e != hipSuccess) return e;
        W4_PF(hipLaunchKernelGGL(pf_resid_norm_kernel, dim3(M), dim3(kThreads), 0, s, m->pf_part, g_o.n_split,
                                 static_cast<size_t>(M) * d, d, m->pf_x, m->ln2[l], eps, m->pf_a));
        e = launch_gemm(g_gu, m->gu_q[l], m->gu_s[l], m->pf_a, M, 2 * f, nullptr, s, m->pf_h);
        if (e != hipSuccess) return e;
        e = launch_gemm(g_dn, m->down_q[l], m->down_s[l], m->pf_h, M, d, m->pf_part, s);
        if (e != hipSuccess) return e;
        const uint16_t *next_w = l + 1 < c.n_layers ? m->ln1[l + 1] : m->lnf;
        W4_PF(hipLaunchKernelGGL(pf_resid_norm_kernel, dim3(M), dim3(kThreads), 0, s, m->pf_part, g_dn.n_split,
                                 static_cast<size_t>(M) * d, d, m->pf_x, next_w, eps, m->pf_a));
    }
    F16Problem hp;
    hp.w = reinterpret_cast<const u32x4 *>(m->lm_head);
    hp.x = reinterpret_cast<const uint32_t *>(m->pf_a + static_cast<size_t>(M - 1) * d);
    hp.n_chunks = d / 8;
    hp.n_rb = m->rb_head;
    hp.n = c.vocab;
    hp.out = m->logits;
    hp.best = &m->state->best;
    W4_PF(hipLaunchKernelGGL(f16_gemv_kernel, dim3(m->rb_head), dim3(kThreads), 0, s, hp));
    W4_PF(hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(1), 0, s, m->state, m->tokens));
#undef W4_PF
    return hipSuccess;
}

// Largest number of work-groups that split one row block, and the checks
// that every work-group's range fits the kernel's LDS areas.
static bool phase_geometry(int T, int nk, int V, int P, int wa, int wb, int &slots, std::string &why,
                           int *max_staged = nullptr) {
    slots = 1;
    const int n_rb = T / nk;
    const Part q = make_part(T, P, wa, wb);
    if (T < P) {
        slots = nk;                       // one work-group per tile
    } else {
        for (int rb = 0; rb < n_rb; ++rb) {
            const int first = part_owner(q, rb * nk);
            const int last = part_owner(q, rb * nk + nk - 1);
            slots = std::max(slots, last - first + 1);
        }
    }
    for (int B = 0; B < P; ++B) {
        const int b = part_start(q, B), e = part_start(q, B + 1);
        if (T >= P && e <= b) { why = "a work-group without tiles"; return false; }
        for (int t = b; t < e; t += std::max(1, (e - b) / 4)) {
            if (part_owner(q, t) != B) { why = "tile owner does not match the ranges"; return false; }
        }
        if (e <= b) continue;
        const int staged = (e - b >= nk ? nk : e - b) * V;   // whole vector or the range's slices
        if (max_staged) *max_staged = std::max(*max_staged, staged);
        if (staged * 2 > kStageBytes) { why = "staged input exceeds LDS"; return false; }
        if (staged > kStageMax * kPkThreads) { why = "staged input exceeds the per-thread batch"; return false; }
        if ((e - 1) / nk - b / nk + 1 > kMaxRbPerWg) { why = "range touches too many row blocks"; return false; }
    }
    return true;
}

static w4_status setup_persistent(w4_model *m) {
    const w4_model_config &c = m->cfg;
    int dev = 0, n_cu = 0, occ = 0;
    W4_HIP(hipGetDevice(&dev));
    W4_HIP(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev));
    int occ8 = 0;
    W4_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, decode_persistent_kernel<false>, kPkThreads, 0));
    W4_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ8, decode_persistent_kernel<true>, kPkThreads, 0));
    occ = std::min(occ, occ8);   // one grid for both variants
    W4_CHECK(occ >= 1 && n_cu >= 1, W4_EHIP, "persistent kernel cannot be resident (occupancy %d)", occ);
    const int P = n_cu * std::min(occ, kPkWgPerCu);
    const int L = c.n_layers, d = c.d_model, f = c.d_ff;
    const int nq = d / kGroup, nf = f / kGroup, nkc = d / 32, no = c.n_q_heads * kHeadDim / kGroup;
    const int rb_q = (c.n_q_heads + 2 * c.n_kv_heads) * kHeadDim / 64, rb_d = d / 64, rb_gu = 2 * f / 64;
    const int rb_lm = (c.vocab + 63) / 64;
    PKParams &pk = m->pk;
    pk = PKParams{};
    pk.P = P;
    std::string why;
    int slots_unused = 0;
    // attention: a work-group per (head, chunk of kPkWaves x att_pps pages), wave
    // v of it taking att_pps pages; at least 2 pages per wave, enough that
    // every (head, chunk) unit has a work-group of its own, and at most 64
    // chunks per head (the O staging merges them a chunk per lane)
    pk.att_pps = std::max({2, (c.max_pages * c.n_q_heads + kPkWaves * P - 1) / (kPkWaves * P),
                           (c.max_pages + kPkWaves * 64 - 1) / (kPkWaves * 64)});
    pk.att_smax = (c.max_pages + kPkWaves * pk.att_pps - 1) / (kPkWaves * pk.att_pps);
    W4_CHECK(c.n_q_heads * pk.att_smax <= P && pk.att_smax <= 64, W4_EINVAL, "too many attention chunks for the grid");
    // two work-groups per CU: the first-dispatched half of the grid gets the
    // larger share of every phase (measured: it gets through a phase faster)
    for (int k = 0; k < 4; ++k) {
        pk.wa[k] = P == 2 * n_cu ? kPkWeights[k][0] : 1;
        pk.wb[k] = P == 2 * n_cu ? kPkWeights[k][1] : 1;
    }
    int staged_max = d;   // the norm phases stage the whole vector
    const bool ok =
        phase_geometry(rb_q * nq, nq, kGroup, P, pk.wa[kPhQ], pk.wb[kPhQ], slots_unused, why, &staged_max) &&
        phase_geometry(rb_d * no, no, kGroup, P, pk.wa[kPhO], pk.wb[kPhO], slots_unused, why, &staged_max) &&
        phase_geometry(rb_gu * nq, nq, kGroup, P, pk.wa[kPhGU], pk.wb[kPhGU], slots_unused, why, &staged_max) &&
        phase_geometry(rb_d * nf, nf, kGroup, P, pk.wa[kPhD], pk.wb[kPhD], slots_unused, why, &staged_max) &&
        phase_geometry(rb_lm * nkc, nkc, 32, P, 1, 1, pk.slots_lm, why);
    m->a8_ok = staged_max <= kA8GroupsPerWave * kPkWaves * kGroup;
    W4_CHECK(ok, W4_EINVAL, "persistent schedule does not fit: %s (grid %d)", why.c_str(), P);
    // normalised inputs are staged whole, one element per thread and batch slot
    W4_CHECK(d <= kStageMax * kPkThreads && d * 2 <= kStageBytes && d <= kEmbChunks * 64 * 8, W4_EINVAL,
             "d_model too large for the persistent step");

    // step-parity blocks: accumulators of every layer, then counters (per
    // layer: 4 phases x groups, one per head; then the embedding counter)
    pk.n_grp = (P + kGW - 1) / kGW;
    pk.cnt_layer = 4 * pk.n_grp + c.n_q_heads;
    pk.acc_q = 0;
    pk.acc_o = pk.acc_q + rb_q * 64;
    pk.acc_gu = pk.acc_o + d;
    pk.acc_d = pk.acc_gu + 2 * f;
    pk.acc_layer = static_cast<size_t>(pk.acc_d + d);
    pk.cnt_off = align256(pk.acc_layer * L * 8);
    pk.par_bytes = pk.cnt_off + align256((static_cast<size_t>(L) * pk.cnt_layer + 1) * kCS * kCRep * 4);

    // library-owned persistent buffers
    const size_t part = static_cast<size_t>(rb_lm) * pk.slots_lm * 64 * 8;
    const int n_ctr = 2 + rb_lm + n_groups(rb_lm);
    const size_t ctr_bytes = align256(static_cast<size_t>(n_ctr) * kCS * 4);
    // residual stream: the embedding row, then per layer after O and after down
    const size_t rstride = align256(static_cast<size_t>(d) * 4) / 4;
    const size_t resid_bytes = rstride * 4 * (2 * static_cast<size_t>(L) + 1);
    const size_t total = align256(sizeof(PKLayer) * L) + align256(sizeof(PKParams)) + align256(resid_bytes) +
                         align256(part) + align256(static_cast<size_t>(c.n_q_heads) * pk.att_smax * 132 * 4) * L +
                         256 + ctr_bytes + 2 * pk.par_bytes;
#ifdef W4_PK_TRACE
    const size_t trace_bytes = static_cast<size_t>(P) * (4 * L + 1) * kTraceSlots * 8;
    W4_HIP(hipMalloc(&m->pk_arena, total + trace_bytes));
    pk.trace = reinterpret_cast<unsigned long long *>(static_cast<char *>(m->pk_arena) + total);
    m->trace_bytes = trace_bytes;
#else
    W4_HIP(hipMalloc(&m->pk_arena, total));
#endif
    W4_HIP(hipMemset(m->pk_arena, 0, total));
    char *b = static_cast<char *>(m->pk_arena);
    m->pk_layers = reinterpret_cast<PKLayer *>(b); b += align256(sizeof(PKLayer) * L);
    m->pk_dev = reinterpret_cast<PKParams *>(b); b += align256(sizeof(PKParams));
    pk.x0 = reinterpret_cast<float *>(b); b += align256(resid_bytes);
    m->resid_stride = rstride;
    pk.partial = reinterpret_cast<double *>(b); b += align256(part);
    pk.att_layer = align256(static_cast<size_t>(c.n_q_heads) * pk.att_smax * 132 * 4) / 4;
    pk.att_part = reinterpret_cast<float *>(b); b += pk.att_layer * 4 * L;
    pk.err = reinterpret_cast<int *>(b); b += 256;
    std::vector<PKLayer> hl(L);
    const size_t kv_layer = layer_kv_elems(m);
    for (int l = 0; l < L; ++l) {
        PKLayer &y = hl[l];
        y.qkv_q = reinterpret_cast<const u32x4 *>(m->qkv_q[l]); y.qkv_s = m->qkv_s[l]; y.qkv_b = m->qkv_bias[l];
        y.o_q = reinterpret_cast<const u32x4 *>(m->o_q[l]); y.o_s = m->o_s[l];
        y.gu_q = reinterpret_cast<const u32x4 *>(m->gu_q[l]); y.gu_s = m->gu_s[l];
        y.dn_q = reinterpret_cast<const u32x4 *>(m->down_q[l]); y.dn_s = m->down_s[l];
        y.ln1 = m->ln1[l]; y.ln2 = m->ln2[l];
        y.kc = m->k_cache + l * kv_layer; y.vc = m->v_cache + l * kv_layer;
        y.xo = pk.x0 + (2 * static_cast<size_t>(l) + 1) * rstride;
        y.xd = pk.x0 + (2 * static_cast<size_t>(l) + 2) * rstride;
    }
    // counters and both parity blocks last and contiguous: reset clears them in one sweep
    pk.ctr = reinterpret_cast<unsigned *>(b); b += ctr_bytes;
    pk.par[0] = b; b += pk.par_bytes;
    pk.par[1] = b; b += pk.par_bytes;
    W4_HIP(hipMemcpy(m->pk_layers, hl.data(), sizeof(PKLayer) * L, hipMemcpyHostToDevice));
    pk.layers = m->pk_layers;
    pk.n_layers = L; pk.d = d; pk.f = f; pk.n_qh = c.n_q_heads; pk.n_kvh = c.n_kv_heads; pk.vocab = c.vocab;
    pk.embed = m->embed; pk.lnf = m->lnf; pk.lm = reinterpret_cast<const u32x4 *>(m->lm_head);
    pk.page_table = m->page_table; pk.tokens = m->tokens; pk.logits = m->logits;
    pk.rope = m->rope;
    pk.st = m->state;
    pk.att_scale_log2 = static_cast<float>(1.4426950408889634 / sqrt(double(kHeadDim)));
    pk.max_pages = c.max_pages;
    pk.dbg_stage = nullptr;
    pk.dbg_stride = std::max(std::max(d, f), c.n_q_heads * kHeadDim);
    pk.eps = static_cast<double>(c.eps);
    pk.c_arr_lm = 2;
    pk.c_grp_lm = 2 + rb_lm;
    const size_t zero_bytes = ctr_bytes + 2 * pk.par_bytes;
    W4_CHECK(zero_bytes / 4 <= static_cast<size_t>(INT32_MAX), W4_EINVAL, "counter region too large");
    m->n_ctr = static_cast<int>(zero_bytes / 4);
    m->pk_grid = P;
    W4_HIP(hipMemcpy(m->pk_dev, &pk, sizeof(PKParams), hipMemcpyHostToDevice));
    return W4_OK;
}

}  // namespace w4

extern "C" w4_status w4_model_create(const w4_model_config *cfg, const w4_model_buffers *buf, w4_model **out) {
    clear_error();
    W4_CHECK(cfg && buf && out, W4_EALIGN, "NULL argument");
    *out = nullptr;
    const w4_model_config &c = *cfg;
    W4_CHECK(c.head_dim == kHeadDim, W4_EINVAL, "head_dim must be 128");
    W4_CHECK(c.n_layers >= 1 && c.n_kv_heads >= 1 && c.n_q_heads >= c.n_kv_heads && c.n_q_heads % c.n_kv_heads == 0 &&
                 gqa_supported(c.n_q_heads / c.n_kv_heads),
             W4_EINVAL, "unsupported head configuration");
    W4_CHECK(c.d_model >= kGroup && c.d_model % kGroup == 0 && c.d_ff >= kGroup && c.d_ff % kGroup == 0, W4_EINVAL,
             "d_model and d_ff must be positive multiples of 128");
    W4_CHECK(c.n_q_heads * kHeadDim >= kGroup, W4_EINVAL, "bad head count");
    W4_CHECK(c.vocab >= 1 && c.max_pages >= 1 && c.eps > 0 && c.theta > 0, W4_EINVAL, "bad vocab/max_pages/eps/theta");
    const void *ptrs[] = {buf->embed, buf->lnf, buf->lm_head, buf->k_cache, buf->v_cache, buf->page_table,
                          buf->free_list, buf->tokens, buf->logits};
    for (const void *p : ptrs) W4_CHECK(p != nullptr, W4_EALIGN, "a model buffer is NULL");
    W4_CHECK(aligned16(buf->lm_head) && aligned16(buf->k_cache) && aligned16(buf->v_cache), W4_EALIGN,
             "lm_head and KV caches must be 16-byte aligned");
    W4_CHECK(reinterpret_cast<uintptr_t>(buf->lnf) % 4 == 0, W4_EALIGN, "lnf must be 4-byte aligned");
    for (int l = 0; l < c.n_layers; ++l) {
        W4_CHECK(buf->qkv_q && buf->qkv_s && buf->qkv_bias && buf->o_q && buf->o_s && buf->gu_q && buf->gu_s &&
                     buf->down_q && buf->down_s && buf->ln1 && buf->ln2,
                 W4_EALIGN, "per-layer pointer arrays must not be NULL");
        W4_CHECK(aligned16(buf->qkv_q[l]) && aligned16(buf->o_q[l]) && aligned16(buf->gu_q[l]) &&
                     aligned16(buf->down_q[l]) && buf->qkv_s[l] && buf->o_s[l] && buf->gu_s[l] && buf->down_s[l] &&
                     buf->qkv_bias[l] && buf->ln1[l] && buf->ln2[l] &&
                     reinterpret_cast<uintptr_t>(buf->ln1[l]) % 4 == 0 && reinterpret_cast<uintptr_t>(buf->ln2[l]) % 4 == 0 &&
                     aligned16(buf->qkv_bias[l]),
                 W4_EALIGN,
                 "layer %d: packed weights and QKV bias must be 16-byte aligned, norm weights 4-byte aligned, others "
                 "non-NULL",
                 l);
    }

    w4_model *m = new w4_model();
    m->cfg = c;
    m->qkv_q.assign(buf->qkv_q, buf->qkv_q + c.n_layers);
    m->qkv_s.assign(buf->qkv_s, buf->qkv_s + c.n_layers);
    m->qkv_bias.assign(buf->qkv_bias, buf->qkv_bias + c.n_layers);
    m->o_q.assign(buf->o_q, buf->o_q + c.n_layers);
    m->o_s.assign(buf->o_s, buf->o_s + c.n_layers);
    m->gu_q.assign(buf->gu_q, buf->gu_q + c.n_layers);
    m->gu_s.assign(buf->gu_s, buf->gu_s + c.n_layers);
    m->down_q.assign(buf->down_q, buf->down_q + c.n_layers);
    m->down_s.assign(buf->down_s, buf->down_s + c.n_layers);
    m->ln1.assign(buf->ln1, buf->ln1 + c.n_layers);
    m->ln2.assign(buf->ln2, buf->ln2 + c.n_layers);
    m->embed = buf->embed;
    m->lnf = buf->lnf;
    m->lm_head = buf->lm_head;
    m->k_cache = buf->k_cache;
    m->v_cache = buf->v_cache;
    m->page_table = buf->page_table;
    m->free_list = buf->free_list;
    m->tokens = buf->tokens;
    m->logits = buf->logits;

    const int d = c.d_model, f = c.d_ff, qd = c.n_q_heads * kHeadDim;
    const int qkv_rows = (c.n_q_heads + 2 * c.n_kv_heads) * kHeadDim;
    m->rb_qkv = (qkv_rows + 63) / 64;
    m->sp_qkv = gemv_split(m->rb_qkv, d / kGroup);
    m->rb_o = (d + 63) / 64;
    m->sp_o = gemv_split(m->rb_o, qd / kGroup);
    m->rb_gu = (2 * f + 63) / 64;
    m->sp_gu = gemv_split(m->rb_gu, d / kGroup);
    m->rb_down = (d + 63) / 64;
    m->sp_down = gemv_split(m->rb_down, f / kGroup);
    m->rb_head = (c.vocab + 63) / 64;
    m->attn_pps = attn_pages_per_split(c.max_pages);
    m->attn_split = attn_n_split(c.max_pages);
    const int G = c.n_q_heads / c.n_kv_heads;

    // counters for up to rb_head row blocks (the largest row-block count) + partials
    size_t part = 0;
    const int rbs[4] = {m->rb_qkv, m->rb_o, m->rb_gu, m->rb_down};
    const int sps[4] = {m->sp_qkv, m->sp_o, m->sp_gu, m->sp_down};
    int max_rb = 1;
    for (int i = 0; i < 4; ++i) {
        part = std::max(part, gemv_partials(rbs[i], sps[i]));
        max_rb = std::max(max_rb, rbs[i]);
    }
    m->ctr_rb = max_rb;
    const size_t max_pos = static_cast<size_t>(c.max_pages) * kPage;
    size_t sizes[10] = {
        align256(sizeof(StepState)),
        align256(static_cast<size_t>(d) * 8),
        align256(static_cast<size_t>(std::max(d, qd)) * 2),
        align256(static_cast<size_t>(qd) * 2),
        align256(static_cast<size_t>(qd) * 2),
        align256(static_cast<size_t>(f) * 2),
        align256(max_pos * 64 * 2 * 8),
        align256(gemv_ws_bytes(max_rb, part)),
        align256(attn_ws_bytes(c.n_kv_heads, G, m->attn_split)),
        align256(static_cast<size_t>(max_rb) * 8) + 256,
    };
    size_t total = 0;
    for (size_t s : sizes) total += s;
    hipError_t e = hipMalloc(&m->arena, total);
    if (e != hipSuccess) {
        model_free(m);
        return fail(W4_EHIP, "hipMalloc(%zu) failed: %s", total, hipGetErrorString(e));
    }
    char *b = static_cast<char *>(m->arena);
    m->state = reinterpret_cast<StepState *>(b); b += sizes[0];
    m->x = reinterpret_cast<double *>(b); b += sizes[1];
    m->a = reinterpret_cast<uint16_t *>(b); b += sizes[2];
    m->qbuf = reinterpret_cast<uint16_t *>(b); b += sizes[3];
    m->o = reinterpret_cast<uint16_t *>(b); b += sizes[4];
    m->h = reinterpret_cast<uint16_t *>(b); b += sizes[5];
    m->rope = reinterpret_cast<double *>(b); b += sizes[6];
    m->gemv_ws = b; b += sizes[7];
    m->attn_ws = b; b += sizes[8];
    m->norm_ctr = reinterpret_cast<unsigned *>(b);
    m->norm_ss = reinterpret_cast<double *>(b + 256); b += sizes[9];
    m->gemv_ws_size = sizes[7];

    // RoPE angles in fp64 on the host: pair i of position p turns by p * theta^(-2i/128)
    std::vector<double> rope(max_pos * 64 * 2);
    for (size_t p = 0; p < max_pos; ++p)
        for (int i = 0; i < 64; ++i) {
            const double inv = pow(c.theta, -2.0 * i / kHeadDim);
            const double phi = static_cast<double>(p) * inv;
            rope[(p * 64 + i) * 2] = cos(phi);
            rope[(p * 64 + i) * 2 + 1] = sin(phi);
        }
    e = hipMemcpy(m->rope, rope.data(), rope.size() * 8, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemset(m->arena, 0, sizes[0]);
    if (e == hipSuccess) e = hipMemset(m->gemv_ws, 0, sizes[7] + sizes[8] + sizes[9]);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&m->cap_stream, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        model_free(m);
        return fail(W4_EHIP, "model setup failed: %s", hipGetErrorString(e));
    }
    w4_status st = setup_prefill(m);
    if (st == W4_OK) st = setup_persistent(m);
    if (st == W4_OK) st = capture(m, false, false, &m->exec[0]);
    if (st == W4_OK) st = capture(m, true, false, &m->exec[1]);
    if (st == W4_OK) st = capture(m, false, true, &m->exec_multi[0]);
    if (st == W4_OK) st = capture(m, true, true, &m->exec_multi[1]);
    if (st != W4_OK) {
        model_free(m);
        return st;
    }
    m->pos = 0;
    m->n_prompt = 0;
    *out = m;
    return W4_OK;
}

#ifdef W4_PK_TRACE
// Trace builds only: copies the persistent kernel's phase timestamps of the
// last step ([grid][4 * n_layers + 1][8] uint64, 100 MHz ticks) to host memory.
extern "C" w4_status w4_model_trace_copy(w4_model *m, void *host, size_t bytes) {
    clear_error();
    W4_CHECK(m != nullptr && host != nullptr && bytes >= m->trace_bytes, W4_EINVAL, "trace needs %zu bytes",
             m ? m->trace_bytes : size_t(0));
    W4_HIP(hipDeviceSynchronize());
    W4_HIP(hipMemcpy(host, m->pk.trace, m->trace_bytes, hipMemcpyDeviceToHost));
    return W4_OK;
}
#endif

extern "C" void w4_model_destroy(w4_model *m) {
    if (m) (void)hipDeviceSynchronize();
    model_free(m);
}

extern "C" w4_status w4_model_reset(w4_model *m, int32_t n_prompt, void *stream) {
    clear_error();
    W4_CHECK(m != nullptr, W4_ESTATE, "no model");
    W4_CHECK(n_prompt >= 1 && n_prompt <= m->cfg.max_pages * kPage, W4_EINVAL, "n_prompt=%d out of range", n_prompt);
    hipLaunchKernelGGL(reset_kernel, dim3(64), dim3(256), 0, static_cast<hipStream_t>(stream), m->state, n_prompt,
                       m->pk.ctr, m->n_ctr, m->pk.err);
    W4_HIP(hipGetLastError());
    m->pos = 0;
    m->n_prompt = n_prompt;
    return W4_OK;
}

extern "C" int32_t w4_model_pos(const w4_model *m) { return m ? m->pos : -1; }

extern "C" int32_t w4_model_launches_per_step(const w4_model *m, uint32_t flags) {
    if (!m) return 0;
    return (flags & W4_MULTI) ? m->launches : 1;
}

extern "C" w4_status decode_step(w4_model *m, int32_t pos, uint32_t flags, void *stream) {
    clear_error();
    W4_CHECK(m != nullptr, W4_ESTATE, "no model");
    W4_CHECK(m->n_prompt >= 1, W4_ESTATE, "w4_model_reset was not called");
    W4_CHECK(pos == m->pos, W4_ESTATE, "position %d out of sequence (model is at %d)", pos, m->pos);
    W4_CHECK(pos < m->cfg.max_pages * kPage, W4_ENOSPC, "position %d beyond the KV pool (%d tokens)", pos,
             m->cfg.max_pages * kPage);
    W4_CHECK(flags <= (W4_EAGER | W4_MULTI | W4_A8), W4_EINVAL, "unknown flags %u", flags);
    const bool boundary = (pos % kPage) == 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool eager = flags & W4_EAGER, multi = flags & W4_MULTI, a8 = flags & W4_A8;
    W4_CHECK(!(a8 && multi), W4_EINVAL, "W4_A8 is a variant of the persistent step, not of W4_MULTI");
    W4_CHECK(!a8 || m->a8_ok, W4_EINVAL, "this model's staged inputs are too long for the int8 variant");
    if (a8 && !eager && !m->exec_a8[0]) {
        w4_status st = capture(m, false, false, &m->exec_a8[0], true);
        if (st == W4_OK) st = capture(m, true, false, &m->exec_a8[1], true);
        if (st != W4_OK) return st;
    }
    if (eager) {
        W4_HIP(multi ? enqueue_step(m, boundary, s) : enqueue_persistent(m, boundary, s, a8));
    } else {
        W4_HIP(hipGraphLaunch((multi ? m->exec_multi : a8 ? m->exec_a8 : m->exec)[boundary ? 1 : 0], s));
    }
    m->pos = pos + 1;
    return W4_OK;
}

extern "C" w4_status w4_model_prefill(w4_model *m, int32_t pos, int32_t n_tokens, void *stream) {
    clear_error();
    W4_CHECK(m != nullptr, W4_ESTATE, "no model");
    W4_CHECK(m->n_prompt >= 1, W4_ESTATE, "w4_model_reset was not called");
    W4_CHECK(pos == m->pos, W4_ESTATE, "position %d out of sequence (model is at %d)", pos, m->pos);
    W4_CHECK(n_tokens >= 1 && n_tokens <= kPrefillMax, W4_EINVAL, "n_tokens=%d outside [1, %d]", n_tokens,
             kPrefillMax);
    W4_CHECK(pos + n_tokens <= m->cfg.max_pages * kPage, W4_ENOSPC, "positions up to %d beyond the KV pool (%d tokens)",
             pos + n_tokens - 1, m->cfg.max_pages * kPage);
    W4_HIP(enqueue_prefill(m, pos, n_tokens, static_cast<hipStream_t>(stream)));
    m->pos = pos + n_tokens;
    return W4_OK;
}

extern "C" w4_status w4_model_kernel_replay(w4_model *m, int32_t kind, int32_t reps, void *stream) {
    clear_error();
    W4_CHECK(m != nullptr, W4_ESTATE, "no model");
    W4_CHECK(reps >= 1, W4_EINVAL, "reps must be positive");
    const w4_model_config &c = m->cfg;
    const int d = c.d_model, f = c.d_ff, qd = c.n_q_heads * kHeadDim;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int r = 0; r < reps; ++r) {
        const int l = r % c.n_layers;
        switch (kind) {
            case W4_KERNEL_GATE_UP:
                W4_HIP(launch_w4(w4_problem(m, m->gu_q[l], m->gu_s[l], m->a, m->rb_gu, m->sp_gu, d),
                                 EpiSwiGLU{m->h, f}, s));
                break;
            case W4_KERNEL_DOWN:
                W4_HIP(launch_w4(w4_problem(m, m->down_q[l], m->down_s[l], m->h, m->rb_down, m->sp_down, f),
                                 EpiResidual{m->x, d}, s));
                break;
            case W4_KERNEL_O:
                W4_HIP(launch_w4(w4_problem(m, m->o_q[l], m->o_s[l], m->o, m->rb_o, m->sp_o, qd),
                                 EpiResidual{m->x, d}, s));
                break;
            case W4_KERNEL_LM_HEAD: {
                F16Problem hp;
                hp.w = reinterpret_cast<const u32x4 *>(m->lm_head);
                hp.x = reinterpret_cast<const uint32_t *>(m->a);
                hp.n_chunks = d / 8;
                hp.n_rb = m->rb_head;
                hp.n = c.vocab;
                hp.out = m->logits;
                hp.best = &m->state->best;
                hipLaunchKernelGGL(f16_gemv_kernel, dim3(m->rb_head), dim3(kThreads), 0, s, hp);
                W4_HIP(hipGetLastError());
                break;
            }
            default:
                return fail(W4_EINVAL, "unknown kernel kind %d", kind);
        }
    }
    return W4_OK;
}

extern "C" w4_status w4_model_status(w4_model *m, int32_t *device_error) {
    clear_error();
    W4_CHECK(m != nullptr && device_error != nullptr, W4_ESTATE, "no model");
    W4_HIP(hipDeviceSynchronize());
    int v = 0;
    W4_HIP(hipMemcpy(&v, m->pk.err, sizeof(int), hipMemcpyDeviceToHost));
    *device_error = v;
    return W4_OK;
}

extern "C" int32_t w4_model_grid(const w4_model *m) { return m ? m->pk_grid : 0; }

// ------------------------------------------------------------ inspection --

extern "C" w4_status w4_model_debug_layout(w4_model *m, w4_debug_layout *out) {
    clear_error();
    W4_CHECK(m != nullptr && out != nullptr, W4_EINVAL, "NULL argument");
    W4_HIP(hipDeviceSynchronize());
    StepState st;
    W4_HIP(hipMemcpy(&st, m->state, sizeof st, hipMemcpyDeviceToHost));
    const PKParams &pk = m->pk;
    out->acc[0] = pk.par[0];
    out->acc[1] = pk.par[1];
    out->acc_layer = static_cast<int64_t>(pk.acc_layer);
    out->acc_q = pk.acc_q;
    out->acc_o = pk.acc_o;
    out->acc_gu = pk.acc_gu;
    out->acc_d = pk.acc_d;
    out->fix_bits = 32;
    out->last_parity = static_cast<int32_t>(st.step & 1u);
    out->resid = pk.x0;
    out->resid_stride = static_cast<int64_t>(m->resid_stride);
    out->att_part = pk.att_part;
    out->att_layer_floats = static_cast<int64_t>(pk.att_layer);
    out->att_smax = pk.att_smax;
    out->att_pages_per_chunk = pk.att_pps * kPkWaves;
    out->stage_stride = pk.dbg_stride;
    return W4_OK;
}

extern "C" size_t w4_model_stage_dump_elems(const w4_model *m) {
    return m ? static_cast<size_t>(4 * m->cfg.n_layers + 1) * static_cast<size_t>(m->pk.dbg_stride) : 0;
}

extern "C" w4_status w4_model_set_stage_dump(w4_model *m, uint16_t *buf) {
    clear_error();
    W4_CHECK(m != nullptr, W4_EINVAL, "no model");
    W4_CHECK(buf == nullptr || (reinterpret_cast<uintptr_t>(buf) & 1) == 0, W4_EALIGN, "bad dump buffer");
    W4_HIP(hipDeviceSynchronize());
    m->pk.dbg_stage = buf;
    W4_HIP(hipMemcpy(m->pk_dev, &m->pk, sizeof(PKParams), hipMemcpyHostToDevice));
    return W4_OK;
}

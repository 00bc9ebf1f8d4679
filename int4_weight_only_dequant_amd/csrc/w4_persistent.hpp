// Persistent decode step for gfx950: the whole 28-layer step in one launch.
//
// The pages' runtime removes per-kernel launch overhead by capturing the
// step as a graph ("Building a Custom LLM Inference Runtime…", section
// "Engineering Challenges" item 2).  On MI355X a graph still pays about 1.6 us
// per node and every kernel boundary drains the HBM pipe, so the step runs
// here as one persistent kernel (still replayed from the two captured graph
// variants) in which waves stream weights continuously:
//
// * Every work-group owns a fixed, contiguous range of "tiles" of every GEMV
//   phase (a tile is 64 packed rows x 128 K elements of int4 codes plus their
//   64 scales, or 64 rows x 32 fp16 elements of the lm_head: four 16-byte
//   loads per lane, one contiguous KiB per wave load); its 4 waves take every
//   4th tile of the range.  Phases run in order QKV -> attention -> O ->
//   gate+up -> down per layer, then the lm_head.
// * Before waiting for a phase's input, a wave issues the loads of its first
//   four tiles of that phase into a register ring; weights do not depend on
//   activations, so HBM keeps streaming while dependencies resolve.
// * A phase's input vector (normalised residual, attention output or SwiGLU
//   output) is staged per work-group in LDS as fp16 and read back with
//   broadcast 16-byte LDS reads.  The RMSNorm is applied while staging: the scale comes
//   from per-row-block sums of squares, summed in a fixed order.
// * Each wave parks its per-row-block sums in LDS; at the end of the phase
//   the work-group adds its 4 waves (fixed order) and publishes one fp64
//   partial per row block.  A row block split across work-groups is reduced
//   by the last one to arrive (partials in fixed slots, summed in slot
//   order), which then
//   runs that row block's epilogue (bias + RoPE + KV append, residual + sum of
//   squares, SwiGLU, or logits + argmax) and bumps the phase's done counter.
// * Cross-wave data is written with device-scope (sc1) stores.  Activation
//   buffers are per layer, so each is written once per launch and read only
//   after its producer signalled: plain (cached) loads cannot see stale lines,
//   because each launch starts with invalidated caches.
// * Every wait is bounded: past a spin limit the wave records an error and
//   every wave bails out, so the grid always drains.  The grid is sized so
//   that all work-groups are resident at once.
#pragma once

#include "w4_gemv.hpp"

namespace w4 {

constexpr int kRing = 4;                 // tiles in flight per wave
constexpr int kMaxRbPerWg = 8;           // row blocks one work-group's range may touch
constexpr int kRedBytes = kMaxRbPerWg * 4 * 64 * 8;
constexpr int kStageBytes = 18432;       // staged fp16 input per work-group
constexpr unsigned kSpinLimit = 1u << 22;

struct StepState {
    int pos;                  // position of the running step
    int n_prompt;             // tokens [0, n_prompt) are teacher-forced
    unsigned long long best;  // argmax key of the step's logits
    unsigned step;            // persistent steps since reset (counter epoch)
    int pad;
};

struct PKLayer {
    const u32x4 *qkv_q; const uint16_t *qkv_s; const uint16_t *qkv_b;
    const u32x4 *o_q; const uint16_t *o_s;
    const u32x4 *gu_q; const uint16_t *gu_s;
    const u32x4 *dn_q; const uint16_t *dn_s;
    const uint16_t *ln1; const uint16_t *ln2;
    uint16_t *kc; uint16_t *vc;            // this layer's KV pools
    uint16_t *q; uint16_t *o; uint16_t *h; // fp16 activations written once per launch
    double *xo; double *xd;                // residual after O / after down
    double *sso; double *ssd;              // per-row-block sums of squares
};

struct PKParams {
    const PKLayer *layers;
    int n_layers, d, f, n_qh, n_kvh, vocab, W;
    const uint16_t *embed; const uint16_t *lnf; const u32x4 *lm;
    const int *page_table; int *tokens; float *logits;
    const double *rope;
    StepState *st;
    double *x0; double *ss0;
    double *partial; float *att_part;
    unsigned *ctr;
    int *err;
    int P;                     // work-groups (all resident)
    int slots_q, slots_o, slots_gu, slots_d, slots_lm;  // partial slot strides per phase
    int att_pps, att_smax;
    float att_scale_log2;
    double eps;
    // counter indices (each counter on its own 128-byte line): per-row-block
    // arrivals, completion groups of 8 row blocks (or heads), per-layer done
    int c_arr_q, c_arr_o, c_arr_gu, c_arr_d, c_arr_lm, c_arr_att, c_layer;
    int c_grp_q, c_grp_o, c_grp_gu, c_grp_d, c_grp_lm, c_grp_att;
};

// Counters sit 128 bytes apart: atomics on one line are serialised at the
// memory side, so unrelated counters must not share a line.
constexpr int kCS = 32;
constexpr int kGrp = 8;         // row blocks (or heads) per completion group

// done counters
enum { kCEmbed = 0, kCLm = 1 };

__host__ __device__ constexpr int n_groups(int n_units) { return (n_units + kGrp - 1) / kGrp; }
enum { kDQkv = 0, kDAttn = 1, kDO = 2, kDGu = 3, kDDn = 4 };

struct Range { int b, e; };

// Work-group B owns tiles [ceil(B T / P), ceil((B+1) T / P)); tile t belongs
// to work-group floor(t P / T).  Inside the range wave v takes every 4th tile.
__device__ __forceinline__ Range wg_range(int B, int T, int P) {
    return {static_cast<int>((static_cast<int64_t>(B) * T + P - 1) / P),
            static_cast<int>((static_cast<int64_t>(B + 1) * T + P - 1) / P)};
}
__device__ __forceinline__ int tile_owner(int t, int T, int P) {
    return static_cast<int>((static_cast<int64_t>(t) * P) / T);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Bounded wait until ctr[idx] reaches target (wrap-safe).  Returns false if
// any wave recorded an error or this wait exceeded the spin limit.
__device__ __noinline__ bool pk_wait(const PKParams &p, int idx, unsigned target) {
    unsigned spins = 0;
    for (;;) {
        const unsigned v = __builtin_amdgcn_readfirstlane(load_agent(p.ctr + idx * kCS));
        if (static_cast<int>(v - target) >= 0) return true;
        if ((spins & 31u) == 31u && __builtin_amdgcn_readfirstlane(load_agent(p.err)) != 0) return false;
        if (++spins > kSpinLimit) {
            if (lane_id() == 0) store_agent(p.err, 1000 + idx);
            return false;
        }
        __builtin_amdgcn_s_sleep(2);
    }
}

// Signal: this wave's prior stores are complete, then bump a counter.
__device__ __forceinline__ unsigned pk_signal(unsigned *ctr) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    unsigned old = 0;
    if (lane_id() == 0) old = atomicAdd(ctr, 1u);
    return __builtin_amdgcn_readfirstlane(old);
}

// A finished unit (row block or head) bumps its group's counter; the last
// unit of a group bumps the phase's done counter.  Returns the done counter's
// previous value if this unit completed a group, else 0xFFFFFFFF.  So a done
// counter receives one atomic per 8 units instead of one per unit.
__device__ __forceinline__ unsigned pk_complete(const PKParams &p, int grp_base, int unit, int n_units,
                                                int done_idx) {
    const int g = unit / kGrp;
    const int gsize = min(kGrp, n_units - g * kGrp);
    const unsigned old = pk_signal(p.ctr + (grp_base + g) * kCS);
    if ((old + 1) % static_cast<unsigned>(gsize) != 0) return 0xFFFFFFFFu;
    unsigned o2 = 0;
    if (lane_id() == 0) o2 = atomicAdd(p.ctr + done_idx * kCS, 1u);
    return __builtin_amdgcn_readfirstlane(o2);
}

// Wave sum in a fixed butterfly order (deterministic).
__device__ __forceinline__ double wave_sum(double v) {
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// RMSNorm scale sqrt(mean(x^2) + eps) from n_rb per-row-block sums of squares.
__device__ __forceinline__ double norm_scale(const double *ss, int n_rb, int d, double eps) {
    double v = 0.0;
    for (int b = lane_id(); b < n_rb; b += 64) v += ss[b];
    return sqrt(wave_sum(v) / d + eps);
}

// ------------------------------------------------------------- tile ring ----

struct Ring {
    u32x4 w[kRing][4];
    uint16_t s[kRing];
};

// int4 tile (rb, g): four 16-byte code loads and the lane's scale
__device__ __forceinline__ void load_w4_tile(Ring &r, int slot, const u32x4 *wq, const uint16_t *ws, int ng,
                                             int t) {
    const int rb = t / ng, g = t - rb * ng, lane = lane_id();
    const u32x4 *src = wq + (static_cast<size_t>(rb) * ng + g) * 256 + lane;
#pragma unroll
    for (int c = 0; c < 4; ++c) r.w[slot][c] = __builtin_nontemporal_load(src + c * 64);
    r.s[slot] = ws[(static_cast<size_t>(rb) * ng + g) * 64 + lane];
}

// fp16 lm_head tile (rb, kc): 32 K elements = four 8-element chunks
__device__ __forceinline__ void load_f16_tile(Ring &r, int slot, const u32x4 *lm, int nkc, int t) {
    const int rb = t / nkc, kc = t - rb * nkc;
    const u32x4 *src = lm + (static_cast<size_t>(rb) * nkc * 4 + kc * 4) * 64 + lane_id();
#pragma unroll
    for (int c = 0; c < 4; ++c) r.w[slot][c] = __builtin_nontemporal_load(src + c * 64);
}

// first kRing tiles of this wave in the work-group range
__device__ __forceinline__ void prefetch_w4(Ring &r, const u32x4 *wq, const uint16_t *ws, int ng, Range rg) {
    const int t0 = rg.b + (static_cast<int>(threadIdx.x) >> 6);
#pragma unroll
    for (int s = 0; s < kRing; ++s)
        if (t0 + 4 * s < rg.e) load_w4_tile(r, s, wq, ws, ng, t0 + 4 * s);
}

__device__ __forceinline__ void prefetch_f16(Ring &r, const u32x4 *lm, int nkc, Range rg) {
    const int t0 = rg.b + (static_cast<int>(threadIdx.x) >> 6);
#pragma unroll
    for (int s = 0; s < kRing; ++s)
        if (t0 + 4 * s < rg.e) load_f16_tile(r, s, lm, nkc, t0 + 4 * s);
}

// ------------------------------------------------------- input staging ----
// Tile t of the work-group range reads V consecutive input elements starting
// at (t % nk) * V.  If the range has at least nk tiles the whole input vector
// is staged (element k at LDS index k); otherwise only the slices of its
// tiles (tile t at LDS index (t - rg.b) * V).  Staging is done by the whole
// work-group, as fp16; the row-block sum area is cleared at the same time.

__device__ __forceinline__ bool stage_whole(Range rg, int nk) { return rg.e - rg.b >= nk; }

__device__ __forceinline__ int stage_off(Range rg, int nk, int V, int t) {
    return (stage_whole(rg, nk) ? t % nk : t - rg.b) * V;
}

__device__ __forceinline__ void stage_begin(double *red, int n_rl) {
    for (int v = threadIdx.x; v < n_rl * 256; v += kThreads) red[v] = 0.0;
}

// Staging issues all of a thread's loads before using any of them (the
// inputs sit in L2 or beyond; one round trip instead of one per element).
constexpr int kStageMax = 16;   // elements per thread (host-checked)

__device__ __forceinline__ void stage_norm(uint16_t *lds, Range rg, int nk, int V, const double *x, double r,
                                           const uint16_t *w) {
    const bool whole = stage_whole(rg, nk);
    const int n = whole ? nk * V : (rg.e - rg.b) * V;
    const double inv_r = 1.0 / r;
    double xv[kStageMax];
    uint16_t wv[kStageMax];
#pragma unroll
    for (int j = 0; j < kStageMax; ++j) {
        const int v = threadIdx.x + j * kThreads;
        if (v < n) {
            const int i = v / V, e = v - i * V;
            const int k = whole ? v : ((rg.b + i) % nk) * V + e;
            xv[j] = x[k];
            wv[j] = w[k];
        }
    }
#pragma unroll
    for (int j = 0; j < kStageMax; ++j) {
        const int v = threadIdx.x + j * kThreads;
        if (v < n) lds[v] = f64_to_f16(xv[j] * inv_r * static_cast<double>(f16_to_f32(wv[j])));
    }
}

__device__ __forceinline__ void stage_plain(uint16_t *lds, Range rg, int nk, int V, const uint16_t *src) {
    const bool whole = stage_whole(rg, nk);
    const int n = whole ? nk * V : (rg.e - rg.b) * V;
    uint16_t sv[kStageMax];
#pragma unroll
    for (int j = 0; j < kStageMax; ++j) {
        const int v = threadIdx.x + j * kThreads;
        if (v < n) {
            const int i = v / V, e = v - i * V;
            sv[j] = src[whole ? v : ((rg.b + i) % nk) * V + e];
        }
    }
#pragma unroll
    for (int j = 0; j < kStageMax; ++j) {
        const int v = threadIdx.x + j * kThreads;
        if (v < n) lds[v] = sv[j];
    }
}

// ---------------------------------------------------- row-block reduction --

// Publish this work-group's sum for row block rb (or finish it alone);
// returns true with the full sum in `total` if this wave must run the
// epilogue.  Called by one wave of the work-group.
// Work-groups contributing to row block rb, and this work-group's slot.
// With T >= P every work-group owns at least one tile, so the owners of the
// row block's tiles are consecutive work-groups; with T < P each tile has its
// own work-group (ranges hold at most one tile).
__device__ __forceinline__ void rb_contrib(int rb, int nk, int T, int P, int B, int &n_contrib, int &slot) {
    const int a = rb * nk;
    if (T >= P) {
        const int first = tile_owner(a, T, P);
        n_contrib = tile_owner(a + nk - 1, T, P) - first + 1;
        slot = B - first;
    } else {
        n_contrib = nk;
        slot = static_cast<int>((static_cast<int64_t>(B) * T + P - 1) / P) - a;   // this work-group's tile
    }
}

__device__ __forceinline__ bool pk_reduce(const PKParams &p, int rb, int nk, int T, int slots, double v,
                                          int arr_base, double &total) {
    unsigned *arr = p.ctr + (arr_base + rb) * kCS;
    int n_contrib, slot;
    rb_contrib(rb, nk, T, p.P, static_cast<int>(blockIdx.x), n_contrib, slot);
    if (n_contrib == 1) {
        total = v;
        return true;
    }
    const int lane = lane_id();
    double *base = p.partial + static_cast<size_t>(rb) * slots * 64 + lane;
    store_agent(base + slot * 64, v);
    const unsigned old = pk_signal(arr);
    if (static_cast<int>(old) != n_contrib - 1) return false;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (lane == 0) store_agent(arr, 0u);
    double s = 0.0;
    int k = 0;
    for (; k + 8 <= n_contrib; k += 8) {
        double a[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) a[u] = load_agent(base + (k + u) * 64);
#pragma unroll
        for (int u = 0; u < 8; ++u) s += a[u];
    }
    for (; k < n_contrib; ++k) s += load_agent(base + k * 64);
    total = s;
    return true;
}

// int4 tile loop of one wave: its tiles rg.b + wave + 4k, consuming the ring
// (already holding the first tiles) and refilling it; per-row-block sums are
// parked in red[rl][wave][lane].
__device__ __forceinline__ void w4_tiles(Ring &r, const u32x4 *wq, const uint16_t *ws, int ng, Range rg,
                                         int rb0, const uint16_t *lds, double *red) {
    const uint32_t m_lo = vreg_const(0x000F000Fu), m_hi = vreg_const(0x00F000F0u), magic = vreg_const(0x64006400u);
    const int wave = wave_id(), lane = lane_id();
    const int n = rg.e - rg.b > wave ? (rg.e - rg.b - wave + 3) / 4 : 0;
    int cur = -1;
    double acc = 0.0;
    for (int k0 = 0; k0 < n; k0 += kRing) {
#pragma unroll
        for (int s = 0; s < kRing; ++s) {
            const int k = k0 + s;
            if (k < n) {
                const int i = wave + 4 * k;          // slot in the work-group range
                const int t = rg.b + i;
                const int rl = t / ng - rb0;
                if (rl != cur) {
                    if (cur >= 0) red[cur * 256 + wave * 64 + lane] = acc;
                    acc = 0.0;
                    cur = rl;
                }
                const u32x4 *xl = reinterpret_cast<const u32x4 *>(lds + stage_off(rg, ng, 128, t));
                float a1 = 0.f, a16 = 0.f;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const u32x4 x0 = xl[c * 4 + 0], x1 = xl[c * 4 + 1], x2 = xl[c * 4 + 2], x3 = xl[c * 4 + 3];
                    const uint32_t xa[4] = {x0.x, x0.y, x0.z, x0.w};
                    const uint32_t xb[4] = {x1.x, x1.y, x1.z, x1.w};
                    const uint32_t xc[4] = {x2.x, x2.y, x2.z, x2.w};
                    const uint32_t xd[4] = {x3.x, x3.y, x3.z, x3.w};
                    dot8v(r.w[s][c].x, xa, a1, a16, m_lo, m_hi, magic);
                    dot8v(r.w[s][c].y, xb, a1, a16, m_lo, m_hi, magic);
                    dot8v(r.w[s][c].z, xc, a1, a16, m_lo, m_hi, magic);
                    dot8v(r.w[s][c].w, xd, a1, a16, m_lo, m_hi, magic);
                }
                acc += static_cast<double>(__builtin_fmaf(a16, 0.0625f, a1)) * static_cast<double>(f16_to_f32(r.s[s]));
                if (k + kRing < n) load_w4_tile(r, s, wq, ws, ng, t + 4 * kRing);
            }
        }
    }
    if (cur >= 0) red[cur * 256 + wave * 64 + lane] = acc;
}

// fp16 (lm_head) tile loop of one wave: fp32 accumulation per row block.
__device__ __forceinline__ void f16_tiles(Ring &r, const u32x4 *lm, int nkc, Range rg, int rb0,
                                          const uint16_t *lds, double *red) {
    const int wave = wave_id(), lane = lane_id();
    const int n = rg.e - rg.b > wave ? (rg.e - rg.b - wave + 3) / 4 : 0;
    int cur = -1;
    float acc0 = 0.f, acc1 = 0.f;
    for (int k0 = 0; k0 < n; k0 += kRing) {
#pragma unroll
        for (int s = 0; s < kRing; ++s) {
            const int k = k0 + s;
            if (k < n) {
                const int i = wave + 4 * k;
                const int t = rg.b + i;
                const int rl = t / nkc - rb0;
                if (rl != cur) {
                    if (cur >= 0) red[cur * 256 + wave * 64 + lane] = static_cast<double>(acc0 + acc1);
                    acc0 = acc1 = 0.f;
                    cur = rl;
                }
                const u32x4 *xl = reinterpret_cast<const u32x4 *>(lds + stage_off(rg, nkc, 32, t));
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const u32x4 xv = xl[c];
                    acc0 = __builtin_amdgcn_fdot2(as_h2(r.w[s][c].x), as_h2(xv.x), acc0, false);
                    acc1 = __builtin_amdgcn_fdot2(as_h2(r.w[s][c].y), as_h2(xv.y), acc1, false);
                    acc0 = __builtin_amdgcn_fdot2(as_h2(r.w[s][c].z), as_h2(xv.z), acc0, false);
                    acc1 = __builtin_amdgcn_fdot2(as_h2(r.w[s][c].w), as_h2(xv.w), acc1, false);
                }
                if (k + kRing < n) load_f16_tile(r, s, lm, nkc, t + 4 * kRing);
            }
        }
    }
    if (cur >= 0) red[cur * 256 + wave * 64 + lane] = static_cast<double>(acc0 + acc1);
}

// ----------------------------------------------------------- epilogues ----

struct PKFinQKV {
    const PKParams *p; const PKLayer *L; int pos; int phys; int n_units; int done_idx;
    __device__ void operator()(int rb, double v) const {
        const int lane = lane_id();
        const int row = rb * 64 + lane;
        const int head = row >> 7, i = (row & 127) >> 1, hi = row & 1, dim = i + 64 * hi;
        const int logical = head * 128 + dim;
        v += static_cast<double>(f16_to_f32(L->qkv_b[logical]));
        const double partner = shfl_xor1(v);
        double out = v;
        if (head < p->n_qh + p->n_kvh) {
            const double c = p->rope[(static_cast<size_t>(pos) * 64 + i) * 2];
            const double s = p->rope[(static_cast<size_t>(pos) * 64 + i) * 2 + 1];
            out = hi ? partner * s + v * c : v * c - partner * s;
        }
        const uint16_t h16 = f64_to_f16(out);
        if (head < p->n_qh) {
            store_agent(L->q + logical, h16);
        } else {
            const int kv = head - p->n_qh;
            const int j = kv < p->n_kvh ? kv : kv - p->n_kvh;
            const size_t off = ((static_cast<size_t>(phys) * p->n_kvh + j) * kPage + (pos & 15)) * kHeadDim + dim;
            store_agent((kv < p->n_kvh ? L->kc : L->vc) + off, h16);
        }
        pk_complete(*p, p->c_grp_q, rb, n_units, done_idx);
    }
};

struct PKFinResid {           // x_new = x_old + v; per-row-block sum of squares
    const PKParams *p; const double *x_old; double *x_new; double *ss; int grp_base; int n_units; int done_idx;
    __device__ void operator()(int rb, double v) const {
        const int row = rb * 64 + lane_id();
        const double xn = x_old[row] + v;
        store_agent(x_new + row, xn);
        const double sq = wave_sum(xn * xn);
        if (lane_id() == 0) store_agent(ss + rb, sq);
        pk_complete(*p, grp_base, rb, n_units, done_idx);
    }
};

struct PKFinSwiGLU {
    const PKParams *p; uint16_t *h; int n_units; int done_idx;
    __device__ void operator()(int rb, double v) const {
        const int lane = lane_id();
        const double u = shfl_xor1(v);
        if ((lane & 1) == 0) store_agent(h + rb * 32 + (lane >> 1), f64_to_f16(v / (1.0 + exp(-v)) * u));
        pk_complete(*p, p->c_grp_gu, rb, n_units, done_idx);
    }
};

struct PKFinLogits {
    const PKParams *p; int n_units; int pos; unsigned epoch; unsigned target;
    __device__ void operator()(int rb, double v) const {
        const int lane = lane_id();
        const int row = rb * 64 + lane;
        const float lg = static_cast<float>(v);
        uint64_t key = 0;
        if (row < p->vocab) {
            p->logits[row] = lg;
            key = argmax_key(lg, row);
        }
        for (int off = 32; off >= 1; off >>= 1) {
            const uint64_t o = __shfl_xor(key, off);
            key = o > key ? o : key;
        }
        if (lane == 0) atomicMax(&p->st->best, static_cast<unsigned long long>(key));
        const unsigned old = pk_complete(*p, p->c_grp_lm, rb, n_units, kCLm);
        if (old + 1 != target) return;
        // the row block that completes the vocabulary finishes the step
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        if (lane == 0) {
            const unsigned long long best = load_agent(&p->st->best);
            const int tok = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best & 0xFFFFFFFFull));
            if (pos + 1 >= p->st->n_prompt) store_agent(p->tokens + pos + 1, tok);
            store_agent(&p->st->best, 0ull);
            store_agent(&p->st->pos, pos + 1);
            store_agent(&p->st->step, epoch + 1);
        }
    }
};

// ----------------------------------------------------------- attention ----
// One wave per (query head, split of pages): lanes = 4 token rows x 16
// eight-dim chunks; each 16-byte load covers 4 tokens of a page.  Splits
// publish (max, sum, 128 weighted-V sums); the last split of a head merges in
// split order and writes fp16 o.

constexpr int kAttPages = 2;   // pages loaded together per wave (8 x 16 B per lane per page)

__device__ __forceinline__ void pk_attention(const PKParams &p, const PKLayer &L, int h, int sp, int n_split,
                                             int ctx, int done_idx) {
    unsigned *arr = p.ctr + (p.c_arr_att + h) * kCS;
    const int lane = lane_id();
    const int ts = lane >> 4, dc = lane & 15;
    const int G = p.n_qh / p.n_kvh, j = h / G;
    const int n_pages = (ctx + kPage - 1) / kPage;
    const int pb = sp * p.att_pps;
    const int pe = min(pb + p.att_pps, n_pages);
    const u32x4 qv = *reinterpret_cast<const u32x4 *>(L.q + h * 128 + dc * 8);
    const size_t slice = static_cast<size_t>(kPage) * kHeadDim;
    float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    // all loads of a chunk of pages are issued together
    auto load_chunk = [&](int c0, u32x4 (&k)[kAttPages][4], u32x4 (&v)[kAttPages][4]) {
#pragma unroll
        for (int pg = 0; pg < kAttPages; ++pg) {
            if (c0 + pg < pe) {
                const int phys = p.page_table[c0 + pg];
                const size_t base = (static_cast<size_t>(phys) * p.n_kvh + j) * slice + ts * kHeadDim + dc * 8;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    k[pg][i] = *reinterpret_cast<const u32x4 *>(L.kc + base + i * 4 * kHeadDim);
                    v[pg][i] = *reinterpret_cast<const u32x4 *>(L.vc + base + i * 4 * kHeadDim);
                }
            }
        }
    };
    u32x4 kn[kAttPages][4], vn[kAttPages][4];
    if (pb < pe) load_chunk(pb, kn, vn);
    for (int c0 = pb; c0 < pe; c0 += kAttPages) {
        u32x4 kcur[kAttPages][4], vcur[kAttPages][4];
#pragma unroll
        for (int pg = 0; pg < kAttPages; ++pg)
#pragma unroll
            for (int i = 0; i < 4; ++i) { kcur[pg][i] = kn[pg][i]; vcur[pg][i] = vn[pg][i]; }
        if (c0 + kAttPages < pe) load_chunk(c0 + kAttPages, kn, vn);
#pragma unroll
        for (int pg = 0; pg < kAttPages; ++pg) {
            if (c0 + pg >= pe) break;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float sc = 0.f;
                sc = __builtin_amdgcn_fdot2(as_h2(qv.x), as_h2(kcur[pg][i].x), sc, false);
                sc = __builtin_amdgcn_fdot2(as_h2(qv.y), as_h2(kcur[pg][i].y), sc, false);
                sc = __builtin_amdgcn_fdot2(as_h2(qv.z), as_h2(kcur[pg][i].z), sc, false);
                sc = __builtin_amdgcn_fdot2(as_h2(qv.w), as_h2(kcur[pg][i].w), sc, false);
                sc = row16_sum(sc) * p.att_scale_log2;
                const int tok = (c0 + pg) * kPage + ts + 4 * i;
                if (tok < ctx) {
                    const float mn = fmaxf(m, sc);
                    const float corr = exp2f(m - mn), pw = exp2f(sc - mn);
                    l = l * corr + pw;
                    const h2 v01 = as_h2(vcur[pg][i].x), v23 = as_h2(vcur[pg][i].y);
                    const h2 v45 = as_h2(vcur[pg][i].z), v67 = as_h2(vcur[pg][i].w);
                    const float vf[8] = {static_cast<float>(v01[0]), static_cast<float>(v01[1]),
                                         static_cast<float>(v23[0]), static_cast<float>(v23[1]),
                                         static_cast<float>(v45[0]), static_cast<float>(v45[1]),
                                         static_cast<float>(v67[0]), static_cast<float>(v67[1])};
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] = acc[e] * corr + pw * vf[e];
                    m = mn;
                }
            }
        }
    }
    // merge the 4 token rows of the wave (lanes 16 and 32 apart)
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
        const float mo = __shfl_xor(m, off), lo = __shfl_xor(l, off);
        const float mn = fmaxf(m, mo);
        const float f0 = m == -INFINITY ? 0.f : exp2f(m - mn);
        const float f1 = mo == -INFINITY ? 0.f : exp2f(mo - mn);
        l = l * f0 + lo * f1;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = acc[e] * f0 + __shfl_xor(acc[e], off) * f1;
        m = mn;
    }
    float *part = p.att_part + (static_cast<size_t>(h) * p.att_smax + sp) * 132;
    if (lane < 16) {
#pragma unroll
        for (int e = 0; e < 8; ++e) store_agent(part + 4 + dc * 8 + e, acc[e]);
    }
    if (lane == 0) {
        store_agent(part, m);
        store_agent(part + 1, l);
    }
    const unsigned old = pk_signal(arr);
    if (static_cast<int>(old) != n_split - 1) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (lane == 0) store_agent(arr, 0u);
    // merge the splits of head h in split order; each batch of 16 splits is
    // loaded with independent loads before any is used
    const float *hb = p.att_part + static_cast<size_t>(h) * p.att_smax * 132;
    float M = -INFINITY, Ls = 0.f, A0 = 0.f, A1 = 0.f;
    for (int s0 = 0; s0 < n_split; s0 += 16) {
        float ms[16], ls[16], a0[16], a1[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            if (s0 + u < n_split) {
                const float *pp = hb + (s0 + u) * 132;
                ms[u] = load_agent(pp);
                ls[u] = load_agent(pp + 1);
                a0[u] = load_agent(pp + 4 + 2 * lane);
                a1[u] = load_agent(pp + 5 + 2 * lane);
            }
        }
        // running rescale across batches (one batch at the usual contexts)
        float Mb = M;
#pragma unroll
        for (int u = 0; u < 16; ++u)
            if (s0 + u < n_split) Mb = fmaxf(Mb, ms[u]);
        const float fr = M == -INFINITY ? 0.f : exp2f(M - Mb);
        Ls *= fr; A0 *= fr; A1 *= fr;
        M = Mb;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            if (s0 + u < n_split && ms[u] != -INFINITY) {
                const float f = exp2f(ms[u] - M);
                Ls += ls[u] * f;
                A0 += a0[u] * f;
                A1 += a1[u] * f;
            }
        }
    }
    const float inv = 1.0f / Ls;
    const uint32_t pair = static_cast<uint32_t>(f32_to_f16(A0 * inv)) | (static_cast<uint32_t>(f32_to_f16(A1 * inv)) << 16);
    store_agent(reinterpret_cast<uint32_t *>(L.o + h * 128) + lane, pair);
    pk_complete(p, p.c_grp_att, h, p.n_qh, done_idx);
}

// ------------------------------------------------------ phase schedule ----
// GEMV phases in order: for each layer QKV, O, gate+up, down; then lm_head.
enum { kPhQ = 0, kPhO = 1, kPhGU = 2, kPhD = 3, kPhLM = 4 };

struct PhaseDesc {
    int kind, l;
    const u32x4 *wq; const uint16_t *ws;
    int nk, V, T, slots, n_rb;
    int arr;                                 // arrival counter base index
    int dep_idx; unsigned dep_target;       // counter that must reach target first
    // staged input: normalised (x, ss, n_ss, w) or plain fp16 (src)
    const double *x; const double *ss; int n_ss; const uint16_t *w;
    const uint16_t *src;
};

__device__ __forceinline__ PhaseDesc phase_desc(const PKParams &p, int ph, unsigned e1) {
    PhaseDesc g{};
    const int d = p.d, nq = d / kGroup, nf = p.f / kGroup, no = p.n_qh * kHeadDim / kGroup;
    const int rb_q = (p.n_qh + 2 * p.n_kvh) * kHeadDim / 64, rb_d = d / 64, rb_gu = 2 * p.f / 64;
    const int L = p.n_layers;
    if (ph >= 4 * L) {
        g.kind = kPhLM; g.l = L - 1;
        g.nk = d / 32; g.V = 32; g.n_rb = (p.vocab + 63) / 64; g.T = g.n_rb * g.nk;
        g.slots = p.slots_lm; g.arr = p.c_arr_lm;
        g.dep_idx = p.c_layer + 5 * (L - 1) + kDDn; g.dep_target = e1 * n_groups(rb_d);
        g.x = p.layers[L - 1].xd; g.ss = p.layers[L - 1].ssd; g.n_ss = rb_d; g.w = p.lnf;
        return g;
    }
    const int l = ph >> 2;
    const PKLayer &Ly = p.layers[l];
    g.kind = ph & 3; g.l = l; g.V = kGroup;
    switch (g.kind) {
        case kPhQ:
            g.wq = Ly.qkv_q; g.ws = Ly.qkv_s; g.nk = nq; g.n_rb = rb_q; g.slots = p.slots_q;
            g.arr = p.c_arr_q;
            if (l == 0) { g.dep_idx = kCEmbed; g.dep_target = e1; g.x = p.x0; g.ss = p.ss0; g.n_ss = 1; }
            else {
                g.dep_idx = p.c_layer + 5 * (l - 1) + kDDn; g.dep_target = e1 * n_groups(rb_d);
                g.x = p.layers[l - 1].xd; g.ss = p.layers[l - 1].ssd; g.n_ss = rb_d;
            }
            g.w = Ly.ln1;
            break;
        case kPhO:
            g.wq = Ly.o_q; g.ws = Ly.o_s; g.nk = no; g.n_rb = rb_d; g.slots = p.slots_o;
            g.arr = p.c_arr_o;
            g.dep_idx = p.c_layer + 5 * l + kDAttn; g.dep_target = e1 * n_groups(p.n_qh);
            g.src = Ly.o;
            break;
        case kPhGU:
            g.wq = Ly.gu_q; g.ws = Ly.gu_s; g.nk = nq; g.n_rb = rb_gu; g.slots = p.slots_gu;
            g.arr = p.c_arr_gu;
            g.dep_idx = p.c_layer + 5 * l + kDO; g.dep_target = e1 * n_groups(rb_d);
            g.x = Ly.xo; g.ss = Ly.sso; g.n_ss = rb_d; g.w = Ly.ln2;
            break;
        default:
            g.wq = Ly.dn_q; g.ws = Ly.dn_s; g.nk = nf; g.n_rb = rb_d; g.slots = p.slots_d;
            g.arr = p.c_arr_d;
            g.dep_idx = p.c_layer + 5 * l + kDGu; g.dep_target = e1 * n_groups(rb_gu);
            g.src = Ly.h;
            break;
    }
    g.T = g.n_rb * g.nk;
    return g;
}

__device__ __forceinline__ void prefetch_phase(Ring &r, const PKParams &p, const PhaseDesc &g) {
    const Range rg = wg_range(blockIdx.x, g.T, p.P);
    if (g.kind == kPhLM) prefetch_f16(r, p.lm, g.nk, rg);
    else prefetch_w4(r, g.wq, g.ws, g.nk, rg);
}

// Epilogue of a finished row block (one wave), by phase kind.
__device__ __noinline__ void pk_finish(const PKParams &p, const PhaseDesc &g, int rb, double v, int pos, int phys,
                                       unsigned epoch) {
    const PKLayer &Ly = p.layers[g.l];
    const int dn = p.c_layer + 5 * g.l;
    switch (g.kind) {
        case kPhQ: {
            PKFinQKV fin{&p, &Ly, pos, phys, g.n_rb, dn + kDQkv};
            fin(rb, v);
            break;
        }
        case kPhO: {
            PKFinResid fin{&p, g.l == 0 ? p.x0 : p.layers[g.l - 1].xd, Ly.xo, Ly.sso, p.c_grp_o, g.n_rb, dn + kDO};
            fin(rb, v);
            break;
        }
        case kPhGU: {
            PKFinSwiGLU fin{&p, Ly.h, g.n_rb, dn + kDGu};
            fin(rb, v);
            break;
        }
        case kPhD: {
            PKFinResid fin{&p, Ly.xo, Ly.xd, Ly.ssd, p.c_grp_d, g.n_rb, dn + kDDn};
            fin(rb, v);
            break;
        }
        default: {
            PKFinLogits fin{&p, g.n_rb, pos, epoch, (epoch + 1) * static_cast<unsigned>(n_groups(g.n_rb))};
            fin(rb, v);
            break;
        }
    }
}

// End of a GEMV phase: the 4 waves' parked sums are added per row block (in
// wave order) and published; finished row blocks run their epilogue.
__device__ __forceinline__ void phase_reduce(const PKParams &p, const PhaseDesc &g, const double *red, int rb0,
                                             int n_rl, int pos, int phys, unsigned epoch) {
    __syncthreads();
    const int wave = wave_id(), lane = lane_id();
    for (int rl = wave; rl < n_rl; rl += 4) {
        const double *rr = red + rl * 256 + lane;
        const double v = ((rr[0] + rr[64]) + rr[128]) + rr[192];
        double tot;
        if (pk_reduce(p, rb0 + rl, g.nk, g.T, g.slots, v, g.arr, tot)) pk_finish(p, g, rb0 + rl, tot, pos, phys, epoch);
    }
    // no trailing barrier: the next phase's LDS writes come after its own
    // work-group-wide barrier
}

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2)))
void decode_persistent_kernel(const PKParams *__restrict__ pp) {
    // parameters live in device memory: functions below take their address,
    // which for a by-value kernel argument would force a copy to scratch
    const PKParams &p = *pp;
    __shared__ __attribute__((aligned(16))) double s_red[kRedBytes / 8];
    __shared__ __attribute__((aligned(16))) uint16_t s_stage[kStageBytes / 2];
    const int wave = wave_id();
    const int B = blockIdx.x;
    const int w = (B << 2) + wave;
    const int W = p.P * 4;
    const int lane = lane_id();

    const int pos = p.st->pos;
    const unsigned epoch = p.st->step;
    const unsigned e1 = epoch + 1;
    const int ctx = pos + 1;
    const int phys = p.page_table[pos >> 4];
    const int L = p.n_layers;
    const int n_pages = (ctx + kPage - 1) / kPage;
    const int n_split = (n_pages + p.att_pps - 1) / p.att_pps;
    const int rb_q = (p.n_qh + 2 * p.n_kvh) * kHeadDim / 64;

    // attention item of this wave (items spread over all waves), if any
    const int n_items_max = p.n_qh * p.att_smax;
    int att_h = -1, att_s = 0;
    {
        const int i0 = static_cast<int>((static_cast<int64_t>(w) * n_items_max + W - 1) / W);
        if (i0 < n_items_max && tile_owner(i0, n_items_max, W) == w) {
            const int hh = i0 / p.att_smax, ss = i0 - hh * p.att_smax;
            if (ss < n_split) { att_h = hh; att_s = ss; }
        }
    }

    // embedding and its sum of squares (one wave); clears the argmax key
    if (w == W - 1) {
        const int d = p.d;
        const int tok = p.tokens[pos];
        const uint16_t *row = p.embed + static_cast<size_t>(tok) * d;
        double sq = 0.0;
        for (int i = lane; i < d; i += 64) {
            const double v = static_cast<double>(f16_to_f32(row[i]));
            store_agent(p.x0 + i, v);
            sq += v * v;
        }
        sq = wave_sum(sq);
        if (lane == 0) {
            store_agent(p.ss0, sq);
            store_agent(&p.st->best, 0ull);
        }
        pk_signal(p.ctr + kCEmbed * kCS);
    }

    Ring ring;
    {
        const PhaseDesc g0 = phase_desc(p, 0, e1);
        prefetch_phase(ring, p, g0);
    }
    bool ok = true;
    const int n_ph = 4 * L + 1;
    for (int ph = 0; ph < n_ph; ++ph) {
        const PhaseDesc g = phase_desc(p, ph, e1);
        const Range rg = wg_range(B, g.T, p.P);
        const bool has_next = ph + 1 < n_ph;
        // attention runs between a layer's QKV and O phases; its waves fill
        // their ring for O only afterwards
        if (g.kind == kPhO && att_h >= 0 && ok) {
            ok = pk_wait(p, p.c_layer + 5 * g.l + kDQkv, e1 * n_groups(rb_q));
            if (ok) {
                // the ring holds nothing this wave still needs: clearing it
                // lets its registers serve the attention loads
                ring = Ring{};
                pk_attention(p, p.layers[g.l], att_h, att_s, n_split, ctx, p.c_layer + 5 * g.l + kDAttn);
                prefetch_phase(ring, p, g);
            }
        }
        const bool next_after_att = has_next && ((ph + 1) & 3) == kPhO && ph + 1 < 4 * L && att_h >= 0;
        if (rg.e > rg.b) {
            ok = ok && pk_wait(p, g.dep_idx, g.dep_target);
            // a failed wait must not strand the other waves at a barrier
            if (__syncthreads_or(!ok)) { ok = false; break; }
            const int rb0 = rg.b / g.nk, n_rl = (rg.e - 1) / g.nk - rb0 + 1;
            stage_begin(s_red, n_rl);
            if (g.src) {
                stage_plain(s_stage, rg, g.nk, g.V, g.src);
            } else {
                const double r = norm_scale(g.ss, g.n_ss, p.d, p.eps);
                stage_norm(s_stage, rg, g.nk, g.V, g.x, r, g.w);
            }
            __syncthreads();
            if (g.kind == kPhLM) f16_tiles(ring, p.lm, g.nk, rg, rb0, s_stage, s_red);
            else w4_tiles(ring, g.wq, g.ws, g.nk, rg, rb0, s_stage, s_red);
            // publish and finish row blocks before issuing the next phase's
            // loads: vmcnt is in order, so any wait on the partial store or
            // the arrival atomic would otherwise also wait for the prefetch
            phase_reduce(p, g, s_red, rb0, n_rl, pos, phys, epoch);
            if (has_next && !next_after_att) prefetch_phase(ring, p, phase_desc(p, ph + 1, e1));
        } else {
            if (!ok) break;
            if (has_next && !next_after_att) prefetch_phase(ring, p, phase_desc(p, ph + 1, e1));
        }
    }
}

}  // namespace w4

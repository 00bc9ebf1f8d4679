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
// * Before waiting for a phase's input, a wave issues the load of its first
//   tile of that phase; weights do not depend on activations, so HBM keeps
//   streaming while dependencies resolve.  In the tile loop each wave keeps
//   one tile in flight while it works on the previous one.
// * Split-K sums of the decoder GEMVs are combined with 64-bit integer atomic
//   adds into per-row accumulators in fixed point (2^-32 units).  Integer
//   addition is associative, so the result does not depend on arrival order
//   (bitwise reproducible) and no work-group has to collect partials.  After
//   its adds are acknowledged a work-group bumps one completion counter (one
//   per group of 8 work-groups, each on its own 128-byte line).
// * Epilogues run on the consumer side while staging the next phase's input
//   in LDS as fp16: residual add + RMSNorm (every consumer rebuilds the whole
//   vector; work-group 0 also stores the residual stream), SwiGLU of the
//   gate/up rows under its down-projection tiles, bias + RoPE for attention,
//   and the merge of the attention splits under its O-projection tiles.  So
//   each phase boundary costs one acknowledged atomic, one counter signal and
//   one round of loads.
// * Accumulators and counters are double-buffered by step parity: a step
//   uses one set and clears the other for the next step.
// * Data read across work-groups (accumulators, attention partials, the
//   residual stream) is read with plain loads, so the work-groups of an XCD
//   share one L2 copy: every such buffer is read only after its producers
//   have signalled, and is written at most once per launch (attention
//   partials are per layer), so no L2 can hold a stale line; each launch
//   starts with invalidated caches.  Counters are polled with device-scope
//   loads.
// * The lm_head keeps per-row-block partials reduced by the last work-group
//   to arrive, which also folds its logits into the step's argmax.
// * Every wait is bounded: past a spin limit the wave records an error and
//   every wave bails out, so the grid always drains.  The grid is sized so
//   that all work-groups are resident at once.
#pragma once

#include "w4_gemv.hpp"

namespace w4 {

// Tiles in flight per wave.  One is best on MI355X: 2048 waves x 4 KiB keep
// about 8 MiB in flight, enough for ~7 TB/s at the loaded latency (~1.2 us);
// deeper rings add no bandwidth, only queueing in front of the latency-bound
// phase hand-overs (measured: 1.70 ms per step at 1, 1.72 at 2, 1.79 at 3,
// 1.87 at 4).
constexpr int kRing = 1;
// Waves per work-group: 4 (two work-groups per CU, weighted ranges) or 8 (one
// per CU).  Measured on the 7B step: 4 waves 1.494 ms, 8 waves 1.499 ms (the
// phase tails shrink with 8, but the waits and the per-work-group reduce
// grow, and attention chunks are twice as long).
#ifndef W4_PK_WAVES
#define W4_PK_WAVES 4
#endif
constexpr int kPkWaves = W4_PK_WAVES;            // waves per work-group
constexpr int kPkThreads = 64 * kPkWaves;        // work-group size
constexpr int kPkWgPerCu = kPkWaves == 4 ? 2 : 1;   // resident work-groups per CU
constexpr int kMaxRbPerWg = kPkWaves == 4 ? 8 : 12;   // row blocks one work-group's range may touch
constexpr int kEmbChunks = 8;            // 16-byte chunks per lane of the embedding row (d <= 4096)
constexpr int kRedBytes = kMaxRbPerWg * kPkWaves * 64 * 8;
constexpr int kStageBytes = 18432;       // staged fp16 input per work-group
constexpr unsigned kSpinLimit = 1u << 22;
constexpr int kGW = 8;                   // work-groups per completion counter
constexpr double kFix = 4294967296.0;    // accumulator units per 1.0
constexpr double kFixInv = 1.0 / 4294967296.0;

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
    float *xo; float *xd;                  // residual stream after O / after down (work-group 0 writes)
};

struct PKParams {
    const PKLayer *layers;
    int n_layers, d, f, n_qh, n_kvh, vocab, W;
    const uint16_t *embed; const uint16_t *lnf; const u32x4 *lm;
    const int *page_table; int *tokens; float *logits;
    const double *rope;
    StepState *st;
    float *x0;                 // embedding row (the layer-0 residual)
    double *partial;
    float *att_part;           // attention split partials, per layer
    size_t att_layer;          // floats per layer of att_part
    unsigned *ctr;             // lm_head arrival and completion counters (128-byte lines)
    int *err;
    int P;                     // work-groups (all resident)
    int slots_lm;              // lm_head partial slot stride
    int att_pps, att_smax;
    float att_scale_log2;
    double eps;
    int c_arr_lm, c_grp_lm;
    // step-parity blocks: int64 accumulators of every layer, then counters
    char *par[2];
    size_t par_bytes;          // bytes per block (a multiple of 16)
    size_t acc_layer;          // accumulators per layer
    int acc_q, acc_o, acc_gu, acc_d;   // row offsets inside a layer
    size_t cnt_off;            // byte offset of the counters in a block
    int n_grp;                 // completion groups of kGW work-groups
    int cnt_layer;             // counters per layer: 4 phases x n_grp, then one per head
    unsigned long long *trace; // [P][phases][kTraceSlots] timestamps (trace builds only)
    int wa[4], wb[4];          // tile-range weights of the grid's first and second half, per phase kind
    int max_pages;             // physical pages of the KV pools
    uint16_t *dbg_stage;       // if set: every GEMV phase's staged fp16 input, [phases][dbg_stride]
    int dbg_stride;
};

// Phase timestamps for profiling (built with -DW4_PK_TRACE; off in the
// product build): wave 0 of each work-group records the 100 MHz real-time
// counter at the points below, per phase.
enum {
    kTrStart = 0,      // top of the phase loop
    kTrWaited = 1,     // dependency wait passed (all waves)
    kTrStaged = 2,     // input staged in LDS (all waves)
    kTrTiles = 3,      // wave 0's tiles done
    kTrSignal = 4,     // accumulators added and completion signalled
    kTrAttBegin = 5,   // attention work-groups: attention started
    kTrAttEnd = 6,     // attention work-groups: chunk published
    kTraceSlots = 8
};
#ifdef W4_PK_TRACE
#define PK_STAMP(ph, k)                                                                                   \
    do {                                                                                                  \
        if (threadIdx.x == 0)                                                                             \
            p.trace[(static_cast<size_t>(blockIdx.x) * (4 * p.n_layers + 1) + (ph)) * kTraceSlots + (k)] = \
                __builtin_amdgcn_s_memrealtime();                                                         \
    } while (0)
#else
#define PK_STAMP(ph, k) \
    do {                \
    } while (0)
#endif

// Counters sit 128 bytes apart: atomics on one line are serialised at the
// memory side, so unrelated counters must not share a line.
constexpr int kCS = 32;
// Copies of every completion counter (phase groups, heads, embedding): a
// signal bumps all copies and work-group B polls copy B % kCRep, so each
// line has 64 pollers (the work-groups of one XCD) instead of 512.  Measured:
// 1572 -> 1554 us per step with 8 copies.
#ifndef W4_PK_CREP
#define W4_PK_CREP 8
#endif
constexpr int kCRep = W4_PK_CREP;
constexpr int kGrp = 8;         // lm_head row blocks per completion group

// done counter of the lm_head
enum { kCLm = 1 };

__host__ __device__ constexpr int n_groups(int n_units) { return (n_units + kGrp - 1) / kGrp; }

// GEMV phases in order: for each layer QKV, O, gate+up, down; then lm_head.
enum { kPhQ = 0, kPhO = 1, kPhGU = 2, kPhD = 3, kPhLM = 4 };

// The layer table through the constant address space: it is read-only for
// the kernel and indexed by uniform layer numbers, so its fields come in by
// scalar loads (a vector load would make the wave wait for every load it has
// in flight, the weight prefetch included).
typedef __attribute__((address_space(4))) const PKLayer *const_layer_ptr;
__device__ __forceinline__ const_layer_ptr pk_layer(const PKParams &p, int l) {
    return (const_layer_ptr)(p.layers) + l;
}

__device__ __forceinline__ long long *pk_acc(const PKParams &p, int par, int l, int off) {
    return reinterpret_cast<long long *>(p.par[par]) + static_cast<size_t>(l) * p.acc_layer + off;
}
// completion counters of (layer, phase kind), one per group; per-head
// attention counters; the embedding counter
__device__ __forceinline__ unsigned *pk_cnt(const PKParams &p, int par, int idx) {
    return reinterpret_cast<unsigned *>(p.par[par] + p.cnt_off) + static_cast<size_t>(idx) * kCS * kCRep;
}
__device__ __forceinline__ unsigned *pk_grp_cnt(const PKParams &p, int par, int l, int kind) {
    return pk_cnt(p, par, l * p.cnt_layer + kind * p.n_grp);
}
__device__ __forceinline__ unsigned *pk_head_cnt(const PKParams &p, int par, int l) {
    return pk_cnt(p, par, l * p.cnt_layer + 4 * p.n_grp);
}
__device__ __forceinline__ unsigned *pk_embed_cnt(const PKParams &p, int par) {
    return pk_cnt(p, par, p.n_layers * p.cnt_layer);
}

struct Range { int b, e; };

// Work-group B owns tiles [ceil(B T / P), ceil((B+1) T / P)); tile t belongs
// to work-group floor(t P / T).  Used for the attention units.
__device__ __forceinline__ Range wg_range(int B, int T, int P) {
    return {static_cast<int>((static_cast<int64_t>(B) * T + P - 1) / P),
            static_cast<int>((static_cast<int64_t>(B + 1) * T + P - 1) / P)};
}
__device__ __forceinline__ int tile_owner(int t, int T, int P) {
    return static_cast<int>((static_cast<int64_t>(t) * P) / T);
}

// Tile ranges of the GEMV phases: contiguous, in work-group order, with
// weights.  Two work-groups share each CU (work-groups are dealt out one per
// CU first, so B and B + P/2 share one), and the first-dispatched one, whose
// waves are older and win instruction and memory issue, gets through a phase
// measurably faster; so the first half of the grid has weight wa and the
// second half wb.  Work-group B owns tiles [start(B), start(B+1)) with
// start(B) = ceil(T cum(B) / W), cum(B) the weight of the work-groups before
// B and W the total; inside the range wave v takes every kPkWaves-th tile.  Phases
// with fewer than 4 tiles per work-group use equal weights.  (The lm_head
// keeps equal weights: see phase_part.)
struct Part {
    int T, P, wa, wb;
};
// Measured on the 7B step (ms per step): 1:1 1.591, 53:47 1.563, 56:44
// 1.551, 59:41 1.537, 62:38 1.510, 66:34 1.506, 70:30 1.522, 75:25 1.595.
#ifndef W4_PK_W_GU
#define W4_PK_W_GU 2, 1
#endif
#ifndef W4_PK_W_D
#define W4_PK_W_D 2, 1
#endif
// weights (first half, second half) per phase kind: QKV, O, gate+up, down
// (QKV and O have fewer than 4 tiles per work-group and use equal ranges).
// Measured with 8-term sums in O and down (us per step): gate+up 2:1 and
// down 2:1 1572, 5:2 and 3:2 1581, 5:2 and 1:1 1600, 3:1 and 1:1 1628.
constexpr int kPkWeights[4][2] = {{1, 1}, {1, 1}, {W4_PK_W_GU}, {W4_PK_W_D}};
__host__ __device__ inline Part make_part(int T, int P, int wa, int wb) {
    return T < 4 * P ? Part{T, P, 1, 1} : Part{T, P, wa, wb};
}
__host__ __device__ inline int64_t part_cum(const Part &q, int B) {
    const int H = q.P / 2;
    return B <= H ? static_cast<int64_t>(q.wa) * B
                  : static_cast<int64_t>(q.wa) * H + static_cast<int64_t>(q.wb) * (B - H);
}
__host__ __device__ inline int part_start(const Part &q, int B) {
    const int64_t W = part_cum(q, q.P);
    return static_cast<int>((static_cast<int64_t>(q.T) * part_cum(q, B) + W - 1) / W);
}
__host__ __device__ inline Range part_range(const Part &q, int B) { return {part_start(q, B), part_start(q, B + 1)}; }
// owner of tile t: the last work-group whose cumulative weight is at most t W / T
__host__ __device__ inline int part_owner(const Part &q, int t) {
    const int64_t W = part_cum(q, q.P);
    const int64_t X = (static_cast<int64_t>(t) * W) / q.T;
    const int H = q.P / 2;
    const int64_t WH = static_cast<int64_t>(q.wa) * H;
    return X < WH ? static_cast<int>(X / q.wa) : H + static_cast<int>((X - WH) / q.wb);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// The thread index behind an empty asm: values derived from it inside the
// phase loop are recomputed where they are used instead of being hoisted out
// of the loop, where they would be spilled (and every reload from scratch
// waits for all outstanding loads, the weight prefetch included).
__device__ __forceinline__ int opaque_tid() {
    int t = static_cast<int>(threadIdx.x);
    asm volatile("" : "+v"(t));
    return t;
}

// Bounded wait (one wave) until counter c_u = base[((b + u) % nk) * kCS]
// reaches its target for every u < n: `want`, or with want == 0 the size of
// completion group u (kGW work-groups, fewer in the last).  Returns false if
// any wave recorded an error or this wait exceeded the spin limit.
__device__ __noinline__ bool pk_wait_cnt(const PKParams &p, const unsigned *base, int n, int b, int nk,
                                         unsigned want, int code) {
    const int lane = lane_id();
    unsigned spins = 0;
    // a lane whose counters have all reached their targets stops polling
    // (counts only grow during a step): fewer loads on the counter lines
    // (measured 1440.8 vs 1442.4 us per step)
    bool sat = false;
    for (;;) {
        bool done = true;
        if (!sat) {
            for (int u = lane; u < n; u += 64) {
                const unsigned target = want ? want : static_cast<unsigned>(min(kGW, p.P - u * kGW));
                done = done && load_agent(base + (static_cast<size_t>((b + u) % nk) * kCRep +
                                                   static_cast<size_t>(blockIdx.x % kCRep)) * kCS) >= target;
            }
            sat = done;
        }
        if (__all(done)) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            return true;
        }
        if ((spins & 31u) == 31u && __builtin_amdgcn_readfirstlane(load_agent(p.err)) != 0) return false;
        if (++spins > kSpinLimit) {
            if (lane == 0) store_agent(p.err, code);
            return false;
        }
        // (polling more slowly while most counters are short of their
        // targets measured slower: 1.491 ms per step at s_sleep 1, 1.499-1.512
        // at 4-16)
        __builtin_amdgcn_s_sleep(1);
    }
}

// Bounded wait until ctr[idx] reaches target (wrap-safe), as above.
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

// Signal: this wave's prior stores and atomics are complete, then bump a counter.
__device__ __forceinline__ unsigned pk_signal(unsigned *ctr) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    unsigned old = 0;
    if (lane_id() == 0) old = atomicAdd(ctr, 1u);
    return __builtin_amdgcn_readfirstlane(old);
}

// Signal on a replicated completion counter: all its copies.
__device__ __forceinline__ void pk_signal_rep(unsigned *ctr) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    if (lane_id() < kCRep) atomicAdd(ctr + lane_id() * kCS, 1u);
}

// A finished lm_head row block bumps its group's counter; the last unit of a
// group bumps the done counter.  Returns the done counter's previous value if
// this unit completed a group, else 0xFFFFFFFF.
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

__device__ __forceinline__ double fix_to_f64(long long a) { return static_cast<double>(a) * kFixInv; }

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
        if (t0 + kPkWaves * s < rg.e) load_w4_tile(r, s, wq, ws, ng, t0 + kPkWaves * s);
}

__device__ __forceinline__ void prefetch_f16(Ring &r, const u32x4 *lm, int nkc, Range rg) {
    const int t0 = rg.b + (static_cast<int>(threadIdx.x) >> 6);
#pragma unroll
    for (int s = 0; s < kRing; ++s)
        if (t0 + kPkWaves * s < rg.e) load_f16_tile(r, s, lm, nkc, t0 + kPkWaves * s);
}

// ------------------------------------------------------- input staging ----
// Tile t reads V consecutive input elements starting at (t % nk) * V.  A
// normalised input is always staged whole (element k at LDS index k); other
// inputs are staged whole if the range has at least nk tiles, otherwise as
// the slices of its tiles (tile t at LDS index (t - rg.b) * V).  Staging is
// done by the whole work-group, as fp16.

__device__ __forceinline__ bool stage_whole(Range rg, int nk) { return rg.e - rg.b >= nk; }

__device__ __forceinline__ void stage_begin(double *red, int n_rl) {
    for (int v = threadIdx.x; v < n_rl * kPkThreads; v += kPkThreads) red[v] = 0.0;
}

// Staging issues all of a thread's loads before using any of them (the
// inputs sit in L2 or beyond; one round trip instead of one per element).
constexpr int kStageMax = kPkWaves == 4 ? 16 : 10;   // elements per thread (host-checked)

// x = x_prev + acc (acc may be null), rounded to the fp32 residual stream;
// RMSNorm with weight w, whole vector to LDS.  Each thread takes element
// pairs (2-byte global loads are slow: the fp16 weights are read two at a
// time).  The sum of squares is fp64 in a fixed order: per thread in pair
// order, within each 16-lane row by DPP, then the 16 row sums of the
// work-group in row order.  If x_out is set the residual is stored there.
typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef long long i64x2 __attribute__((ext_vector_type(2)));
constexpr int kPairMax = kStageMax / 2;

__device__ __forceinline__ double dpp_f64(double v, int ctrl_q) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    int lo, hi;
    switch (ctrl_q) {   // the DPP control must be a constant
        case 0: lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(b), 0xB1, 0xF, 0xF, false);
                hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), 0xB1, 0xF, 0xF, false); break;
        case 1: lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(b), 0x4E, 0xF, 0xF, false);
                hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), 0x4E, 0xF, 0xF, false); break;
        case 2: lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(b), 0x141, 0xF, 0xF, false);   // row_half_mirror
                hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), 0x141, 0xF, 0xF, false); break;
        default: lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(b), 0x140, 0xF, 0xF, false);  // row_mirror
                 hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), 0x140, 0xF, 0xF, false); break;
    }
    return __builtin_bit_cast(double, (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                                          static_cast<uint32_t>(lo));
}

// Sum over each 16-lane row (every lane of the row gets it): pairs, quads,
// halves, rows.
__device__ __forceinline__ double row16_sum_f64(double v) {
    v += dpp_f64(v, 0);
    v += dpp_f64(v, 1);
    v += dpp_f64(v, 2);
    v += dpp_f64(v, 3);
    return v;
}

__device__ __forceinline__ void stage_resid_norm(uint16_t *lds, double *wsum, int d, const float *x_prev,
                                                 const long long *acc, const uint16_t *w, double eps,
                                                 float *x_out) {
    const int np = d / 2;
    const int tid = opaque_tid();
    float2 xv[kPairMax];
    i64x2 av[kPairMax];
    uint32_t wv[kPairMax];
#pragma unroll
    for (int j = 0; j < kPairMax; ++j) {
        const int q = tid + j * kPkThreads;
        if (q < np) {
            xv[j] = reinterpret_cast<const float2 *>(x_prev)[q];
            wv[j] = reinterpret_cast<const uint32_t *>(w)[q];
            if (acc) av[j] = reinterpret_cast<const i64x2 *>(acc)[q];
            else av[j] = i64x2{0, 0};
        }
    }
    double sq = 0.0;
#pragma unroll
    for (int j = 0; j < kPairMax; ++j) {
        const int q = tid + j * kPkThreads;
        if (q < np) {
            xv[j].x = static_cast<float>(static_cast<double>(xv[j].x) + fix_to_f64(av[j].x));
            xv[j].y = static_cast<float>(static_cast<double>(xv[j].y) + fix_to_f64(av[j].y));
            sq += static_cast<double>(xv[j].x) * xv[j].x;
            sq += static_cast<double>(xv[j].y) * xv[j].y;
        }
    }
    sq = row16_sum_f64(sq);
    if ((tid & 15) == 0) wsum[tid >> 4] = sq;
    __syncthreads();
    double ss = 0.0;
#pragma unroll
    for (int r = 0; r < kPkThreads / 16; ++r) ss += wsum[r];
    // the scaling itself runs in fp32: its rounding (a few 2^-24) sits far
    // below the fp16 rounding of the result
    const float inv_r = static_cast<float>(1.0 / sqrt(ss / d + eps));
#pragma unroll
    for (int j = 0; j < kPairMax; ++j) {
        const int q = tid + j * kPkThreads;
        if (q < np) {
            if (x_out) {   // device-scope stores: read by other XCDs after the next signal
                store_agent(x_out + 2 * q, xv[j].x);
                store_agent(x_out + 2 * q + 1, xv[j].y);
            }
            const uint32_t lo = f32_to_f16(xv[j].x * inv_r * f16_to_f32(wv[j] & 0xFFFFu));
            const uint32_t hi = f32_to_f16(xv[j].y * inv_r * f16_to_f32(wv[j] >> 16));
            reinterpret_cast<uint32_t *>(lds)[q] = lo | (hi << 16);
        }
    }
}

// h = silu(gate) * up from the gate/up accumulators (gate row 2k, up row
// 2k + 1 for element k; one 16-byte load per element), for the tiles of the
// range; element pairs per thread so LDS takes 4-byte writes.
__device__ __forceinline__ void stage_swiglu(uint16_t *lds, Range rg, int nk, int V, const long long *acc) {
    const bool whole = stage_whole(rg, nk);
    const int n = whole ? nk * V : (rg.e - rg.b) * V;
    const int tid = opaque_tid();
    i64x2 a0[kPairMax], a1[kPairMax];
#pragma unroll
    for (int j = 0; j < kPairMax; ++j) {
        const int v = 2 * (tid + j * kPkThreads);
        if (v < n) {
            const int i = v / V, e = v - i * V;            // V is even: the pair stays in one tile
            const int k = whole ? v : ((rg.b + i) % nk) * V + e;
            a0[j] = reinterpret_cast<const i64x2 *>(acc)[k];
            a1[j] = reinterpret_cast<const i64x2 *>(acc)[k + 1];
        }
    }
#pragma unroll
    for (int j = 0; j < kPairMax; ++j) {
        const int v = 2 * (tid + j * kPkThreads);
        if (v < n) {
            // exp in fp32 (relative error ~1e-7, far below the fp16 rounding
            // of h); a double exp's coefficient table would be hoisted out
            // of the phase loop and spilled
            uint32_t h2v[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const i64x2 a = u ? a1[j] : a0[j];
                const double g = fix_to_f64(a.x), up = fix_to_f64(a.y);
                const double ex = static_cast<double>(__expf(static_cast<float>(-g)));
                h2v[u] = f64_to_f16(g / (1.0 + ex) * up);
            }
            reinterpret_cast<uint32_t *>(lds)[v >> 1] = h2v[0] | (h2v[1] << 16);
        }
    }
}

// Wave reductions by DPP within 16-lane rows, then lane reads across rows
// (a fixed order: the results do not depend on timing).
__device__ __forceinline__ int dpp_i32(int v, int ctrl_q) {
    switch (ctrl_q) {   // the DPP control must be a constant
        case 0: return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
        case 1: return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
        case 2: return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);   // row_half_mirror
        default: return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
    }
}
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int c = 0; c < 4; ++c) v = fmaxf(v, __builtin_bit_cast(float, dpp_i32(__builtin_bit_cast(int, v), c)));
    const int b = __builtin_bit_cast(int, v);
    return fmaxf(fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)),
                       __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))),
                 fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)),
                       __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48))));
}
__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
    for (int c = 0; c < 4; ++c) v += dpp_i32(v, c);
    return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
           (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int c = 0; c < 4; ++c) v += __builtin_bit_cast(float, dpp_i32(__builtin_bit_cast(int, v), c));
    const int b = __builtin_bit_cast(int, v);
    return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
           (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
}

// Attention output of the heads under the range's O-projection tiles (a
// 128-element K group is one head).  A wave per head: lane c holds chunk c's
// (max, sum) (at most 64 chunks, host-checked), the wave takes the maximum
// and each chunk's weight; every lane then adds the chunks' weighted sums for
// its dims 2 lane, 2 lane + 1 in chunk order, kAttMergeBatch chunks' loads
// in flight at once.  (Measured per step at context 520 and 8192: batches of
// 24 1536/1780 us with 224 spilled SGPRs, 16 1480/1739, 8 1444/1720 with 59
// and no spilled VGPRs; the former merge, every lane taking the weights of 16
// chunks per batch itself, 1504/1863 with 20 spilled VGPRs.)
constexpr int kAttMergeBatch = 8;
__device__ __forceinline__ void stage_attn(uint16_t *lds, Range rg, int nk, const float *att_part, int att_smax,
                                           int n_split) {
    const bool whole = stage_whole(rg, nk);
    const int n_u = whole ? nk : rg.e - rg.b;
    const int lane = opaque_tid() & 63;
    for (int u = wave_id(); u < n_u; u += kPkWaves) {
        const int h = whole ? u : (rg.b + u) % nk;
        const float *hb = att_part + static_cast<size_t>(h) * att_smax * 132;
        float2 ml = make_float2(-INFINITY, 0.f);
        if (lane < n_split) ml = *reinterpret_cast<const float2 *>(hb + lane * 132);
        float A0 = 0.f, A1 = 0.f, w = 0.f, Ls = 0.f;
        for (int s0 = 0; s0 < n_split; s0 += kAttMergeBatch) {
            float2 aa[kAttMergeBatch];
#pragma unroll
            for (int q = 0; q < kAttMergeBatch; ++q)
                if (s0 + q < n_split) aa[q] = *reinterpret_cast<const float2 *>(hb + (s0 + q) * 132 + 4 + 2 * lane);
            if (s0 == 0) {
                const float M = wave_max_f32(ml.x);
                w = ml.x == -INFINITY ? 0.f : exp2f(ml.x - M);
                Ls = wave_sum_f32(w * ml.y);
            }
#pragma unroll
            for (int q = 0; q < kAttMergeBatch; ++q) {
                if (s0 + q < n_split) {
                    const float wq = __builtin_bit_cast(
                        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), s0 + q));
                    A0 += wq * aa[q].x;
                    A1 += wq * aa[q].y;
                }
            }
        }
        const float inv = 1.0f / Ls;
        const uint32_t pair =
            static_cast<uint32_t>(f32_to_f16(A0 * inv)) | (static_cast<uint32_t>(f32_to_f16(A1 * inv)) << 16);
        reinterpret_cast<uint32_t *>(lds + u * 128)[lane] = pair;
    }
}

// ---------------------------------------------------- row-block reduction --

// Work-groups contributing to lm_head row block rb, and this work-group's
// slot.  With T >= P every work-group owns at least one tile, so the owners
// of the row block's tiles are consecutive work-groups; with T < P each tile
// has its own work-group (ranges hold at most one tile).
__device__ __forceinline__ void rb_contrib(int rb, int nk, const Part &q, int B, int &n_contrib, int &slot) {
    const int a = rb * nk;
    if (q.T >= q.P) {
        const int first = part_owner(q, a);
        n_contrib = part_owner(q, a + nk - 1) - first + 1;
        slot = B - first;
    } else {
        n_contrib = nk;
        slot = part_start(q, B) - a;   // this work-group's tile
    }
}

// Publish this work-group's lm_head sum for row block rb (or finish it
// alone); returns true with the full sum in `total` if this wave must run the
// epilogue.  Called by one wave of the work-group.
__device__ __forceinline__ bool pk_reduce(const PKParams &p, int rb, int nk, int T, int slots, double v,
                                          int arr_base, double &total) {
    unsigned *arr = p.ctr + (arr_base + rb) * kCS;
    int n_contrib, slot;
    rb_contrib(rb, nk, make_part(T, p.P, 1, 1), static_cast<int>(blockIdx.x), n_contrib, slot);
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
// parked in red[rl][wave][lane].  kShort: short 8-term sums added in fp64
// (the down projection, whose inputs, SwiGLU outputs, reach 10^2 and more),
// else one chained fp32 accumulation per group (QKV, O, gate+up: measured
// within the GEMV tolerance on the layer tests; O's attention-output inputs
// of up to about 30 gave 4.7e-4 at the 8192-token context against 2e-3).
template <bool kShort>
__device__ __forceinline__ void w4_tiles(Ring &r, const u32x4 *wq, const uint16_t *ws, int ng, Range rg,
                                         bool whole, int rb0, const uint16_t *lds, double *red) {
    const uint32_t m_lo = vreg_const(0x000F000Fu), m_hi = vreg_const(0x00F000F0u), magic = vreg_const(0x64006400u), magic_hi = vreg_const(0x54005400u);
    const int wave = wave_id(), lane = lane_id();
    const int n = rg.e - rg.b > wave ? (rg.e - rg.b - wave + kPkWaves - 1) / kPkWaves : 0;
    int cur = -1;
    double acc = 0.0;
    for (int k0 = 0; k0 < n; k0 += kRing) {
#pragma unroll
        for (int s = 0; s < kRing; ++s) {
            const int k = k0 + s;
            if (k < n) {
                const int i = wave + kPkWaves * k;   // slot in the work-group range
                const int t = rg.b + i;
                const int rl = t / ng - rb0;
                if (rl != cur) {
                    if (cur >= 0) red[cur * kPkThreads + wave * 64 + lane] = acc;
                    acc = 0.0;
                    cur = rl;
                }
                const u32x4 *xl = reinterpret_cast<const u32x4 *>(lds + (whole ? t % ng : i) * 128);
                double gs;
                if constexpr (kShort) {
                    gs = 0.0;
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const u32x4 x0 = xl[c * 4 + 0], x1 = xl[c * 4 + 1], x2 = xl[c * 4 + 2], x3 = xl[c * 4 + 3];
                        const uint32_t xa[4] = {x0.x, x0.y, x0.z, x0.w};
                        const uint32_t xb[4] = {x1.x, x1.y, x1.z, x1.w};
                        const uint32_t xc[4] = {x2.x, x2.y, x2.z, x2.w};
                        const uint32_t xd[4] = {x3.x, x3.y, x3.z, x3.w};
                        gs += static_cast<double>(dot8v_short(r.w[s][c].x, xa, m_lo, m_hi, magic, magic_hi));
                        gs += static_cast<double>(dot8v_short(r.w[s][c].y, xb, m_lo, m_hi, magic, magic_hi));
                        gs += static_cast<double>(dot8v_short(r.w[s][c].z, xc, m_lo, m_hi, magic, magic_hi));
                        gs += static_cast<double>(dot8v_short(r.w[s][c].w, xd, m_lo, m_hi, magic, magic_hi));
                    }
                } else {
                    float a1 = 0.f, a2 = 0.f;
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const u32x4 x0 = xl[c * 4 + 0], x1 = xl[c * 4 + 1], x2 = xl[c * 4 + 2], x3 = xl[c * 4 + 3];
                        const uint32_t xa[4] = {x0.x, x0.y, x0.z, x0.w};
                        const uint32_t xb[4] = {x1.x, x1.y, x1.z, x1.w};
                        const uint32_t xc[4] = {x2.x, x2.y, x2.z, x2.w};
                        const uint32_t xd[4] = {x3.x, x3.y, x3.z, x3.w};
                        dot8v(r.w[s][c].x, xa, a1, a2, m_lo, m_hi, magic, magic_hi);
                        dot8v(r.w[s][c].y, xb, a1, a2, m_lo, m_hi, magic, magic_hi);
                        dot8v(r.w[s][c].z, xc, a1, a2, m_lo, m_hi, magic, magic_hi);
                        dot8v(r.w[s][c].w, xd, a1, a2, m_lo, m_hi, magic, magic_hi);
                    }
                    gs = static_cast<double>(a1 + a2);
                }
                acc += gs * static_cast<double>(f16_to_f32(r.s[s]));
                if (k + kRing < n) load_w4_tile(r, s, wq, ws, ng, t + kPkWaves * kRing);
            }
        }
    }
    if (cur >= 0) red[cur * kPkThreads + wave * 64 + lane] = acc;
}

// ------------------------------------------- int8 activations (W4_A8) --
// The int8-activation variant of the step ("Building a Custom LLM Inference
// Runtime…", section "Engineering Challenges" item 3; "The Architecture of
// Modern Inference…", section "Three Critical Engineering Challenges" item
// 3): each int4 GEMV's staged fp16 input is quantised per group of 128 in
// the staging area itself, as w4a8_quantize_act does: scale s = max|x| / 127
// in fp32, codes round-half-even(x / s) in fp32 clamped to [-127, 127] (an
// all-zero group: scale 0, zero codes), plus each group's code sum.  Codes
// of group u go to bytes 128 u .. 128 u + 127 of the staging area in the
// order the int4 words pair them with (words (e0, e4, e1, e5), (e2, e6, e3,
// e7) per block of 8), the scales and sums after them.
constexpr int kA8GroupsPerWave = 8;                       // host-checked: at most 32 staged groups
// scales and sums sit past the fp16 input of the largest staging (written
// while the fp16 is still being read)
constexpr int kA8ScaleOff = kA8GroupsPerWave * kPkWaves * 256;
constexpr int kA8SumOff = kA8ScaleOff + kA8GroupsPerWave * kPkWaves * 4;
static_assert(kA8SumOff + kA8GroupsPerWave * kPkWaves * 4 <= kStageBytes, "int8 staging fits the stage area");

// Wave-wide max and sum: within each 16-lane row by DPP (as row16_sum),
// then the four row results by readlane (a shuffle through LDS per step
// measured about 4 us per phase on the step).
// ng staged groups of 128 fp16 (group u at element 128 u), in place; wave w
// takes groups w, w + 4, ...; lane holds elements 2 lane, 2 lane + 1.  All
// reads finish before the barrier, all writes come after it (the codes of a
// group overlap the fp16 of lower groups).  Ends with a barrier.
__device__ __forceinline__ void stage_quant_a8(uint16_t *lds, int ng) {
    const int wave = wave_id(), lane = lane_id();
    unsigned char *cb = reinterpret_cast<unsigned char *>(lds);
    uint32_t code2[kA8GroupsPerWave];
#pragma unroll
    for (int k = 0; k < kA8GroupsPerWave; ++k) {
        const int u = wave + kPkWaves * k;
        code2[k] = 0u;
        if (u < ng) {
            const uint32_t pr = reinterpret_cast<const uint32_t *>(lds)[u * 64 + lane];
            const float x0 = f16_to_f32(static_cast<uint16_t>(pr & 0xFFFFu));
            const float x1 = f16_to_f32(static_cast<uint16_t>(pr >> 16));
            const float amax = wave_max_f32(fmaxf(fabsf(x0), fabsf(x1)));
            const float sc = amax / 127.0f;                        // IEEE division, as the oracle's float32
            int c0 = 0, c1 = 0;
            if (sc != 0.f) {
                c0 = static_cast<int>(fminf(fmaxf(rintf(x0 / sc), -127.f), 127.f));
                c1 = static_cast<int>(fminf(fmaxf(rintf(x1 / sc), -127.f), 127.f));
            }
            code2[k] = static_cast<uint32_t>(c0 & 0xFF) | (static_cast<uint32_t>(c1 & 0xFF) << 8);
            const int sm = wave_sum_i32(c0 + c1);
            if (lane == 0) {
                reinterpret_cast<float *>(cb + kA8ScaleOff)[u] = sc;
                reinterpret_cast<int *>(cb + kA8SumOff)[u] = sm;
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kA8GroupsPerWave; ++k) {
        const int u = wave + kPkWaves * k;
        if (u < ng) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int e = 2 * lane + h, blk = e >> 3, r = e & 7;
                const int word = 2 * blk + ((r >> 1) & 1), byte = ((r & 1) << 1) | (r >> 2);
                cb[u * 128 + word * 4 + byte] = static_cast<unsigned char>((code2[k] >> (8 * h)) & 0xFFu);
            }
        }
    }
    __syncthreads();
}

// int4 x int8 tile loop of one wave (same walk as w4_tiles): per tile the
// integer dot product of the unsigned nibbles (q + 8) with the codes, minus
// 8 x the group's code sum, times the activation and weight scales in fp64.
__device__ __forceinline__ void w4_tiles_a8(Ring &r, const u32x4 *wq, const uint16_t *ws, int ng, Range rg,
                                            bool whole, int rb0, const uint16_t *lds, double *red) {
    // lane index and nibble mask produced here behind empty asm rather than
    // as plain expressions the compiler may hoist out of the phase loop: with
    // the plain forms this kernel spilled 40 VGPRs (8 of them the weight ring)
    const int wave = wave_id(), lane = opaque_tid() & 63;
    const uint32_t m4 = vreg_const(0x0F0F0F0Fu);
    const int n = rg.e - rg.b > wave ? (rg.e - rg.b - wave + kPkWaves - 1) / kPkWaves : 0;
    const unsigned char *cb = reinterpret_cast<const unsigned char *>(lds);
    int cur = -1;
    double acc = 0.0;
    for (int k0 = 0; k0 < n; k0 += kRing) {
#pragma unroll
        for (int s = 0; s < kRing; ++s) {
            const int k = k0 + s;
            if (k < n) {
                const int i = wave + kPkWaves * k;
                const int t = rg.b + i;
                const int rl = t / ng - rb0;
                if (rl != cur) {
                    if (cur >= 0) red[cur * kPkThreads + wave * 64 + lane] = acc;
                    acc = 0.0;
                    cur = rl;
                }
                const int gx = whole ? t % ng : i;
                const u32x4 *xc = reinterpret_cast<const u32x4 *>(cb + gx * 128);
                int dot = 0;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const u32x4 xa = xc[2 * c], xb = xc[2 * c + 1];
                    const uint32_t wv[4] = {r.w[s][c].x, r.w[s][c].y, r.w[s][c].z, r.w[s][c].w};
                    const uint32_t xl[4] = {xa.x, xa.z, xb.x, xb.z}, xh[4] = {xa.y, xa.w, xb.y, xb.w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        dot = __builtin_amdgcn_sdot4(static_cast<int>(wv[q] & m4), static_cast<int>(xl[q]), dot,
                                                     false);
                        dot = __builtin_amdgcn_sdot4(static_cast<int>((wv[q] >> 4) & m4),
                                                     static_cast<int>(xh[q]), dot, false);
                    }
                }
                const float sx = reinterpret_cast<const float *>(cb + kA8ScaleOff)[gx];
                const int sumc = reinterpret_cast<const int *>(cb + kA8SumOff)[gx];
                acc += static_cast<double>(dot - 8 * sumc) * static_cast<double>(sx) *
                       static_cast<double>(f16_to_f32(r.s[s]));
                if (k + kRing < n) load_w4_tile(r, s, wq, ws, ng, t + kPkWaves * kRing);
            }
        }
    }
    if (cur >= 0) red[cur * kPkThreads + wave * 64 + lane] = acc;
}

// fp16 (lm_head) tile loop of one wave: fp32 accumulation per row block; the
// normalised input is staged whole.  (Two or three tiles in flight per wave
// instead of one measured the same, 1.495-1.497 ms per step: the phase
// already streams at about 6.1 TB/s.)
__device__ __forceinline__ void f16_tiles(Ring &r, const u32x4 *lm, int nkc, Range rg, int rb0,
                                          const uint16_t *lds, double *red) {
    const int wave = wave_id(), lane = lane_id();
    const int n = rg.e - rg.b > wave ? (rg.e - rg.b - wave + kPkWaves - 1) / kPkWaves : 0;
    int cur = -1;
    float acc0 = 0.f, acc1 = 0.f;
    for (int k0 = 0; k0 < n; k0 += kRing) {
#pragma unroll
        for (int s = 0; s < kRing; ++s) {
            const int k = k0 + s;
            if (k < n) {
                const int i = wave + kPkWaves * k;
                const int t = rg.b + i;
                const int rl = t / nkc - rb0;
                if (rl != cur) {
                    if (cur >= 0) red[cur * kPkThreads + wave * 64 + lane] = static_cast<double>(acc0 + acc1);
                    acc0 = acc1 = 0.f;
                    cur = rl;
                }
                const u32x4 *xl = reinterpret_cast<const u32x4 *>(lds + (t % nkc) * 32);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const u32x4 xv = xl[c];
                    acc0 = __builtin_amdgcn_fdot2(as_h2(r.w[s][c].x), as_h2(xv.x), acc0, false);
                    acc1 = __builtin_amdgcn_fdot2(as_h2(r.w[s][c].y), as_h2(xv.y), acc1, false);
                    acc0 = __builtin_amdgcn_fdot2(as_h2(r.w[s][c].z), as_h2(xv.z), acc0, false);
                    acc1 = __builtin_amdgcn_fdot2(as_h2(r.w[s][c].w), as_h2(xv.w), acc1, false);
                }
                if (k + kRing < n) load_f16_tile(r, s, lm, nkc, t + kPkWaves * kRing);
            }
        }
    }
    if (cur >= 0) red[cur * kPkThreads + wave * 64 + lane] = static_cast<double>(acc0 + acc1);
}

// ------------------------------------------------------- lm_head epilogue --

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
// A work-group per (query head, chunk of W x pps pages, W its waves); its
// wave v takes pages [chunk * W pps + v pps, + pps).  In a wave, lanes = 4 token rows x 16
// eight-dim chunks; each 16-byte load covers 4 tokens of a page.  The K/V
// pages are requested before waiting for the QKV phase (they hold earlier
// tokens only).  The query (and, for the running position, that token's key
// and value) comes straight from the QKV accumulators: bias, RoPE and the
// fp16 rounding are applied here, and the wave holding the running position
// of the first query head of a kv group writes the new key and value into
// the cache for later steps.  The waves' online-softmax states are merged
// through LDS in wave order; the chunk's (max, sum, 128 weighted-V sums) is
// published and the head's counter bumped; the O projection merges chunks.

constexpr int kAttPages = 2;   // pages loaded together per wave (8 x 16 B per lane per page)

// The query of head h (and, with kv, the running token's key and value of kv
// head j) from the QKV accumulators, as fp16 into LDS: sq[128], sk[128],
// sv[128].  Thread t < 128 takes query dim t and value dim t, thread t >= 128
// key dim t - 128: bias, then RoPE (dims i and i + 64 pair up; in QKV row
// order they are rows 2i and 2i + 1 of the head), in fp64.  Every load is
// issued before any is used.
__device__ __forceinline__ void qkv_to_lds(const PKParams &p, const long long *acc, const uint16_t *bias, int h,
                                           int j, int pos, bool kv, uint16_t *sq, uint16_t *sk, uint16_t *sv) {
    const int t = opaque_tid();
    if (t >= 256) return;                          // 128 query dims, 128 key (or value) dims
    const int d = t & 127, i = d & 63, hi = d >> 6;
    const bool first = t < 128;
    const bool rot = first || kv;                  // q, or k when wanted
    const int head = first ? h : p.n_qh + j;
    const int hv = p.n_qh + p.n_kvh + j;
    long long a_own = 0, a_par = 0, a_v = 0;
    uint16_t b_own = 0, b_par = 0, b_v = 0;
    double c = 0.0, sn = 0.0;
    if (rot) {
        a_own = acc[head * 128 + 2 * i + hi];
        a_par = acc[head * 128 + 2 * i + (hi ^ 1)];
        b_own = bias[head * 128 + d];
        b_par = bias[head * 128 + (d ^ 64)];
        c = p.rope[(static_cast<size_t>(pos) * 64 + i) * 2];
        sn = p.rope[(static_cast<size_t>(pos) * 64 + i) * 2 + 1];
    }
    if (first && kv) {
        a_v = acc[hv * 128 + 2 * i + hi];
        b_v = bias[hv * 128 + d];
    }
    if (rot) {
        const double v = fix_to_f64(a_own) + static_cast<double>(f16_to_f32(b_own));
        const double pa = fix_to_f64(a_par) + static_cast<double>(f16_to_f32(b_par));
        const double r = hi ? pa * sn + v * c : v * c - pa * sn;
        (first ? sq : sk)[d] = f64_to_f16(r);
    }
    if (first && kv) sv[d] = f64_to_f16(fix_to_f64(a_v) + static_cast<double>(f16_to_f32(b_v)));
}

// K and V of pages [c0, min(c0 + kAttPages, pe)) for this lane
__device__ __forceinline__ void att_load(const PKParams &p, const_layer_ptr L, int j, int c0, int pe, int ts, int dc,
                                         u32x4 (&k)[kAttPages][4], u32x4 (&v)[kAttPages][4]) {
    const size_t slice = static_cast<size_t>(kPage) * kHeadDim;
    // the page table is read-only for the step: scalar loads, all issued
    // before the K/V loads that depend on them
    const const_u32_ptr pt = as_const(reinterpret_cast<const uint32_t *>(p.page_table));
    int phy[kAttPages];
#pragma unroll
    for (int pg = 0; pg < kAttPages; ++pg)
        phy[pg] = c0 + pg < pe ? static_cast<int>(pt[__builtin_amdgcn_readfirstlane(c0 + pg)]) : 0;
#pragma unroll
    for (int pg = 0; pg < kAttPages; ++pg) {
        if (c0 + pg < pe) {
            const size_t base = (static_cast<size_t>(phy[pg]) * p.n_kvh + j) * slice + ts * kHeadDim + dc * 8;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                k[pg][i] = *reinterpret_cast<const u32x4 *>(L->kc + base + i * 4 * kHeadDim);
                v[pg][i] = *reinterpret_cast<const u32x4 *>(L->vc + base + i * 4 * kHeadDim);
            }
        }
    }
}

// Returns false if the wait for the QKV phase failed (all waves agree).
__device__ __forceinline__ bool pk_attention(const PKParams &p, const_layer_ptr L, const unsigned *q_done,
                                             const long long *acc_q, float *att_part, unsigned *head_cnt, int h,
                                             int c, int n_split, int ctx, int phys, float *s_att, uint16_t *s_qkv,
                                             int code) {
    const int lane = opaque_tid() & 63, wave = wave_id();
    const int ts = lane >> 4, dc = lane & 15;
    const int G = p.n_qh / p.n_kvh, j = h / G;
    const int pos = ctx - 1;
    const int n_pages = (ctx + kPage - 1) / kPage;
    const int pb = (c * kPkWaves + wave) * p.att_pps;
    const int pe = min(pb + p.att_pps, n_pages);
    u32x4 kc[kAttPages][4], vc[kAttPages][4];
    if (pb < pe) att_load(p, L, j, pb, pe, ts, dc, kc, vc);
    bool ok = true;
    if (wave == 0) ok = pk_wait_cnt(p, q_done, p.n_grp, 0, p.n_grp, 0, code);
    if (__syncthreads_or(!ok)) return false;

    const bool has_cur = pb < pe && pe == n_pages;   // this wave holds the running position
    const bool last_chunk = c == n_split - 1;       // the work-group holding the running position
    uint16_t *sq = s_qkv, *sk = s_qkv + 128, *sv = s_qkv + 256;
    qkv_to_lds(p, acc_q, L->qkv_b, h, j, pos, last_chunk, sq, sk, sv);
    __syncthreads();
    const u32x4 qv = *reinterpret_cast<const u32x4 *>(sq + dc * 8);
    u32x4 knew{}, vnew{};
    if (has_cur) {
        knew = *reinterpret_cast<const u32x4 *>(sk + dc * 8);
        vnew = *reinterpret_cast<const u32x4 *>(sv + dc * 8);
    }
    // the first query head of a kv group writes the new key and value
    if (last_chunk && h == j * G && wave == 0 && lane < 32) {
        const size_t off = ((static_cast<size_t>(phys) * p.n_kvh + j) * kPage + (pos & 15)) * kHeadDim + (lane & 15) * 8;
        const u32x4 val = *reinterpret_cast<const u32x4 *>((lane < 16 ? sk : sv) + (lane & 15) * 8);
        *reinterpret_cast<u32x4 *>((lane < 16 ? L->kc : L->vc) + off) = val;
    }
    float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int c0 = pb; c0 < pe; c0 += kAttPages) {
        if (c0 != pb) att_load(p, L, j, c0, pe, ts, dc, kc, vc);
        // all scores of the resident pages first (independent dot products
        // and row reductions), then one rescale and one accumulation pass
        float sc[kAttPages][4];
        float mb = -INFINITY;
#pragma unroll
        for (int pg = 0; pg < kAttPages; ++pg) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = (c0 + pg) * kPage + ts + 4 * i;
                // the running token's key is not in the cache yet
                const u32x4 kk = tok == pos ? knew : kc[pg][i];
                float v = 0.f;
                v = __builtin_amdgcn_fdot2(as_h2(qv.x), as_h2(kk.x), v, false);
                v = __builtin_amdgcn_fdot2(as_h2(qv.y), as_h2(kk.y), v, false);
                v = __builtin_amdgcn_fdot2(as_h2(qv.z), as_h2(kk.z), v, false);
                v = __builtin_amdgcn_fdot2(as_h2(qv.w), as_h2(kk.w), v, false);
                v = row16_sum(v) * p.att_scale_log2;
                const bool valid = c0 + pg < pe && tok < ctx;
                sc[pg][i] = valid ? v : -INFINITY;
                mb = fmaxf(mb, sc[pg][i]);
            }
        }
        const float mn = fmaxf(m, mb);
        if (mn != -INFINITY) {
            const float corr = exp2f(m - mn);
            l *= corr;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] *= corr;
#pragma unroll
            for (int pg = 0; pg < kAttPages; ++pg) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (sc[pg][i] == -INFINITY) continue;
                    const int tok = (c0 + pg) * kPage + ts + 4 * i;
                    const u32x4 vv = tok == pos ? vnew : vc[pg][i];
                    const float pw = exp2f(sc[pg][i] - mn);
                    l += pw;
                    const h2 v01 = as_h2(vv.x), v23 = as_h2(vv.y);
                    const h2 v45 = as_h2(vv.z), v67 = as_h2(vv.w);
                    const float vf[8] = {static_cast<float>(v01[0]), static_cast<float>(v01[1]),
                                         static_cast<float>(v23[0]), static_cast<float>(v23[1]),
                                         static_cast<float>(v45[0]), static_cast<float>(v45[1]),
                                         static_cast<float>(v67[0]), static_cast<float>(v67[1])};
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] += pw * vf[e];
                }
            }
            m = mn;
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
    // merge the waves in wave order through LDS: [wave][m, l, 128 dims]
    float *sw = s_att + wave * 130;
    if (lane < 16) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sw[2 + dc * 8 + e] = acc[e];
    }
    if (lane == 0) { sw[0] = m; sw[1] = l; }
    __syncthreads();
    if (wave == 0) {
        float M = -INFINITY;
#pragma unroll
        for (int v = 0; v < kPkWaves; ++v) M = fmaxf(M, s_att[v * 130]);
        float Ls = 0.f, A0 = 0.f, A1 = 0.f;
#pragma unroll
        for (int v = 0; v < kPkWaves; ++v) {
            const float mv = s_att[v * 130];
            if (mv != -INFINITY) {
                const float f = exp2f(mv - M);
                Ls += s_att[v * 130 + 1] * f;
                A0 += s_att[v * 130 + 2 + 2 * lane] * f;
                A1 += s_att[v * 130 + 3 + 2 * lane] * f;
            }
        }
        float *part = att_part + (static_cast<size_t>(h) * p.att_smax + c) * 132;
        store_agent(part + 4 + 2 * lane, A0);
        store_agent(part + 5 + 2 * lane, A1);
        if (lane == 0) {
            store_agent(part, M);
            store_agent(part + 1, Ls);
        }
        pk_signal_rep(head_cnt + h * kCS * kCRep);
    }
    return true;
}

// ------------------------------------------------------ phase schedule ----

enum { kStNorm = 0, kStSwiGLU = 1, kStAttn = 2 };

struct PhaseDesc {
    int kind, l;
    const u32x4 *wq; const uint16_t *ws;
    int nk, V, T, n_rb;
    // input dependency: counters base[((b + u) % nk) * kCS] for the units u
    // of the range (per-tile units, dep_all: all dep_n) must reach dep_want
    // (0: completion-group sizes)
    const unsigned *dep; int dep_n; unsigned dep_want; bool dep_all;
    // staging: normalised residual (x_prev + acc_in, weight w, store to
    // x_out), SwiGLU of acc_in, or merged attention
    int stage;
    const float *x_prev; const long long *acc_in; const uint16_t *w; float *x_out;
    long long *acc_out;       // this phase's accumulators
    unsigned *done;           // this phase's completion counters
};

__device__ __forceinline__ PhaseDesc phase_desc(const PKParams &p, int ph, int par, int n_split) {
    PhaseDesc g{};
    const int d = p.d, nq = d / kGroup, nf = p.f / kGroup, no = p.n_qh * kHeadDim / kGroup;
    const int rb_q = (p.n_qh + 2 * p.n_kvh) * kHeadDim / 64, rb_d = d / 64, rb_gu = 2 * p.f / 64;
    const int L = p.n_layers;
    g.dep_all = true;
    g.dep_n = p.n_grp;
    g.dep_want = 0;
    g.stage = kStNorm;
    if (ph >= 4 * L) {
        g.kind = kPhLM; g.l = L - 1;
        g.nk = d / 32; g.V = 32; g.n_rb = (p.vocab + 63) / 64; g.T = g.n_rb * g.nk;
        g.dep = pk_grp_cnt(p, par, L - 1, kPhD);
        g.x_prev = pk_layer(p, L - 1)->xo; g.acc_in = pk_acc(p, par, L - 1, p.acc_d); g.w = p.lnf;
        g.x_out = pk_layer(p, L - 1)->xd;
        return g;
    }
    const int l = ph >> 2;
    const const_layer_ptr Ly = pk_layer(p, l);
    g.kind = ph & 3; g.l = l; g.V = kGroup;
    g.done = pk_grp_cnt(p, par, l, g.kind);
    switch (g.kind) {
        case kPhQ:
            g.wq = Ly->qkv_q; g.ws = Ly->qkv_s; g.nk = nq; g.n_rb = rb_q;
            g.acc_out = pk_acc(p, par, l, p.acc_q);
            if (l == 0) {
                g.dep = pk_embed_cnt(p, par); g.dep_n = 1; g.dep_want = 1;
                g.x_prev = p.x0;
            } else {
                g.dep = pk_grp_cnt(p, par, l - 1, kPhD);
                g.x_prev = pk_layer(p, l - 1)->xo; g.acc_in = pk_acc(p, par, l - 1, p.acc_d);
                g.x_out = pk_layer(p, l - 1)->xd;
            }
            g.w = Ly->ln1;
            break;
        case kPhO:          // a 128-element K group of the O projection is one head
            g.wq = Ly->o_q; g.ws = Ly->o_s; g.nk = no; g.n_rb = rb_d;
            g.acc_out = pk_acc(p, par, l, p.acc_o);
            g.dep = pk_head_cnt(p, par, l); g.dep_n = p.n_qh; g.dep_want = static_cast<unsigned>(n_split);
            g.dep_all = false;
            g.stage = kStAttn;
            break;
        case kPhGU:
            g.wq = Ly->gu_q; g.ws = Ly->gu_s; g.nk = nq; g.n_rb = rb_gu;
            g.acc_out = pk_acc(p, par, l, p.acc_gu);
            g.dep = pk_grp_cnt(p, par, l, kPhO);
            g.x_prev = l == 0 ? p.x0 : pk_layer(p, l - 1)->xd; g.acc_in = pk_acc(p, par, l, p.acc_o);
            g.w = Ly->ln2; g.x_out = Ly->xo;
            break;
        default:
            g.wq = Ly->dn_q; g.ws = Ly->dn_s; g.nk = nf; g.n_rb = rb_d;
            g.acc_out = pk_acc(p, par, l, p.acc_d);
            g.dep = pk_grp_cnt(p, par, l, kPhGU);
            g.stage = kStSwiGLU; g.acc_in = pk_acc(p, par, l, p.acc_gu);
            break;
    }
    g.T = g.n_rb * g.nk;
    return g;
}

// Tile ranges of a phase: weighted for the decoder GEMVs; equal for the
// lm_head, a long phase in which the two work-groups of a CU share it evenly
// (measured: with the 2:1 weights the first half's lm_head tiles took 167 us
// against 99 us for the second half).
__device__ __forceinline__ Part phase_part(const PKParams &p, const PhaseDesc &g) {
    return g.kind == kPhLM ? make_part(g.T, p.P, 1, 1) : make_part(g.T, p.P, p.wa[g.kind], p.wb[g.kind]);
}

__device__ __forceinline__ void prefetch_phase(Ring &r, const PKParams &p, const PhaseDesc &g) {
    const Range rg = part_range(phase_part(p, g), blockIdx.x);
    if (g.kind == kPhLM) prefetch_f16(r, p.lm, g.nk, rg);
    else prefetch_w4(r, g.wq, g.ws, g.nk, rg);
}

// Inspection hook (off unless a dump buffer is set): the phase's staged fp16
// input at its element positions.  A normalised input, or one staged whole,
// comes from work-group 0; slices staged per tile are written by every
// work-group that staged them (identical values).
__device__ __noinline__ void pk_dump_stage(uint16_t *dst, const uint16_t *lds, int n_whole, int rb, int re, int nk,
                                           int V) {
    if (n_whole > 0) {
        if (blockIdx.x != 0) return;
        for (int i = threadIdx.x; i < n_whole; i += kPkThreads) dst[i] = lds[i];
        return;
    }
    const int n = (re - rb) * V;
    for (int i = threadIdx.x; i < n; i += kPkThreads) {
        const int u = i / V, e = i - u * V;
        dst[((rb + u) % nk) * V + e] = lds[i];
    }
}

__device__ __noinline__ void pk_finish_lm(const PKParams &p, const PhaseDesc &g, int rb, double v, int pos,
                                          unsigned epoch) {
    PKFinLogits fin{&p, g.n_rb, pos, epoch, (epoch + 1) * static_cast<unsigned>(n_groups(g.n_rb))};
    fin(rb, v);
}

// End of a GEMV phase: the 4 waves' parked sums are added per row block (in
// wave order).  Decoder phases add them to the accumulators and bump the
// work-group's completion counter once every wave's adds are acknowledged;
// the lm_head reduces per row block and runs its epilogue.
__device__ __forceinline__ void phase_reduce(const PKParams &p, const PhaseDesc &g, const double *red, int rb0,
                                             int n_rl, int pos, unsigned epoch) {
    __syncthreads();
    const int wave = wave_id(), lane = lane_id();
    for (int rl = wave; rl < n_rl; rl += kPkWaves) {
        const double *rr = red + rl * kPkThreads + lane;
        double v = rr[0];
#pragma unroll
        for (int u = 1; u < kPkWaves; ++u) v += rr[u * 64];   // wave order
        if (g.kind == kPhLM) {
            double tot;
            if (pk_reduce(p, rb0 + rl, g.nk, g.T, p.slots_lm, v, p.c_arr_lm, tot))
                pk_finish_lm(p, g, rb0 + rl, tot, pos, epoch);
        } else {
            __hip_atomic_fetch_add(g.acc_out + (rb0 + rl) * 64 + lane, __double2ll_rn(v * kFix), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (g.kind != kPhLM) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (wave == 0) pk_signal_rep(g.done + (blockIdx.x / kGW) * kCS * kCRep);
    }
    // no trailing barrier: the next phase's LDS writes come after its own
    // work-group-wide barrier
}

// kA8: the int8-activation variant (every int4 GEMV's input quantised in
// staging, integer dot products); the lm_head stays fp16.
template <bool kA8>
__global__ __attribute__((amdgpu_flat_work_group_size(kPkThreads, kPkThreads), amdgpu_waves_per_eu(2)))
void decode_persistent_kernel(const PKParams *__restrict__ pp) {
    // parameters live in device memory: functions below take their address,
    // which for a by-value kernel argument would force a copy to scratch
    const PKParams &p = *pp;
    __shared__ __attribute__((aligned(16))) double s_red[kRedBytes / 8];
    __shared__ __attribute__((aligned(16))) uint16_t s_stage[kStageBytes / 2];
    __shared__ double s_wsum[kPkThreads / 16];
    const int wave = wave_id();
    const int B = blockIdx.x;
    const int w = B * kPkWaves + wave;
    const int W = p.P * kPkWaves;
    const int lane = lane_id();

    const int pos = p.st->pos;
    const unsigned epoch = p.st->step;
    const unsigned e1 = epoch + 1;
    const int par = static_cast<int>(e1 & 1u);
    const int ctx = pos + 1;
    const int phys = p.page_table[pos >> 4];
    // A failed step leaves its error word set: later steps do nothing until
    // the model is reset.  A token id or page outside its table would be an
    // access out of bounds: every work-group sees the same values and leaves.
    {
        const int tok0 = p.tokens[pos];
        int bad = 0;
        if (load_agent(p.err) != 0) bad = -1;
        else if (phys < 0 || phys >= p.max_pages) bad = 5000;
        else if (tok0 < 0 || tok0 >= p.vocab) bad = 5001;
        if (bad != 0) {
            if (bad > 0 && B == 0 && threadIdx.x == 0) store_agent(p.err, bad);
            return;
        }
    }
    const int L = p.n_layers;
    const int n_pages = (ctx + kPage - 1) / kPage;
    // attention chunks of kPkWaves x att_pps pages per head at this context
    const int n_split = (n_pages + kPkWaves * p.att_pps - 1) / (kPkWaves * p.att_pps);

    // attention unit (head, chunk) of this work-group, if any.  The query
    // heads of one kv head and chunk read the same K/V pages: they go to
    // work-groups of one XCD (work-groups are dealt to the 8 XCDs
    // round-robin, so B % 8 is the XCD), where all but the first read of a
    // page hit that XCD's L2.  If the XCD slots cannot hold every group, the
    // units are spread over all work-groups instead.
    const int n_units_max = p.n_qh * p.att_smax;
    int att_h = -1, att_s = 0;
    {
        const int G = p.n_qh / p.n_kvh;
        const int n_grp = p.n_kvh * p.att_smax;              // (kv head, chunk) groups
        const int slots = p.P / 8;                            // work-groups per XCD
        if (p.P % 8 == 0 && ((n_grp + 7) / 8) * G <= slots) {
            const int x = B & 7, slot = B >> 3;
            const int grp = (slot / G) * 8 + x, k = slot % G;
            if (grp < n_grp) {
                const int jj = grp / p.att_smax, ss = grp - jj * p.att_smax;
                if (ss < n_split) { att_h = jj * G + k; att_s = ss; }
            }
        } else {
            const int i0 = static_cast<int>((static_cast<int64_t>(B) * n_units_max + p.P - 1) / p.P);
            if (i0 < n_units_max && tile_owner(i0, n_units_max, p.P) == B) {
                const int hh = i0 / p.att_smax, ss = i0 - hh * p.att_smax;
                if (ss < n_split) { att_h = hh; att_s = ss; }
            }
        }
    }

    Ring ring;
    prefetch_phase(ring, p, phase_desc(p, 0, par, n_split));

    // embedding (one wave); clears the argmax key.  Every 16-byte load of the
    // row is issued before any value is stored (a store between loads would
    // keep the next load behind it: one memory round trip per element).
    if (w == W - 1) {
        const int n8 = p.d / 8;                      // 16-byte chunks of the row (host: d <= 4096)
        const int tok = p.tokens[pos];
        const u32x4 *row = reinterpret_cast<const u32x4 *>(p.embed + static_cast<size_t>(tok) * p.d);
        u32x4 v[kEmbChunks];
#pragma unroll
        for (int u = 0; u < kEmbChunks; ++u)
            if (lane + 64 * u < n8) v[u] = row[lane + 64 * u];
#pragma unroll
        for (int u = 0; u < kEmbChunks; ++u) {
            const int c = lane + 64 * u;
            if (c < n8) {
                const uint32_t wd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    store_agent(p.x0 + c * 8 + 2 * e, f16_to_f32(static_cast<uint16_t>(wd[e] & 0xFFFFu)));
                    store_agent(p.x0 + c * 8 + 2 * e + 1, f16_to_f32(static_cast<uint16_t>(wd[e] >> 16)));
                }
            }
        }
        if (lane == 0) store_agent(&p.st->best, 0ull);
        pk_signal_rep(pk_embed_cnt(p, par));
    }


    bool ok = true;
    const int n_ph = 4 * L + 1;
    for (int ph = 0; ph < n_ph; ++ph) {
        const PhaseDesc g = phase_desc(p, ph, par, n_split);
        const Range rg = part_range(phase_part(p, g), B);
        const bool has_next = ph + 1 < n_ph;
        PK_STAMP(ph, kTrStart);
        // attention runs between a layer's QKV and O phases; its waves fill
        // their ring for O only afterwards
        if (g.kind == kPhO && att_h >= 0) {
            if (!ok) break;
            // the ring holds nothing this wave still needs: clearing it
            // lets its registers serve the attention loads
            ring = Ring{};
            PK_STAMP(ph, kTrAttBegin);
            ok = pk_attention(p, pk_layer(p, g.l), pk_grp_cnt(p, par, g.l, kPhQ), pk_acc(p, par, g.l, p.acc_q),
                              p.att_part + g.l * p.att_layer, pk_head_cnt(p, par, g.l), att_h, att_s, n_split, ctx,
                              phys, reinterpret_cast<float *>(s_red), s_stage, 2000 + g.l);
            PK_STAMP(ph, kTrAttEnd);
            if (!ok) break;
            prefetch_phase(ring, p, g);
        }
        const bool next_after_att = has_next && ((ph + 1) & 3) == kPhO && ph + 1 < 4 * L && att_h >= 0;
        if (rg.e > rg.b) {
            const bool whole = g.stage == kStNorm || stage_whole(rg, g.nk);
            if (ok && wave == 0) {
                if (g.dep_all || whole)
                    ok = pk_wait_cnt(p, g.dep, g.dep_n, 0, g.dep_n, g.dep_want, 3000 + ph);
                else
                    ok = pk_wait_cnt(p, g.dep, rg.e - rg.b, rg.b, g.nk, g.dep_want, 3000 + ph);
            }
            // a failed wait must not strand the other waves at a barrier
            if (__syncthreads_or(!ok)) { ok = false; break; }
            PK_STAMP(ph, kTrWaited);
            const int rb0 = rg.b / g.nk, n_rl = (rg.e - 1) / g.nk - rb0 + 1;
            stage_begin(s_red, n_rl);
            if (g.stage == kStNorm)
                stage_resid_norm(s_stage, s_wsum, p.d, g.x_prev, g.acc_in, g.w, p.eps, B == 0 ? g.x_out : nullptr);
            else if (g.stage == kStSwiGLU)
                stage_swiglu(s_stage, rg, g.nk, g.V, g.acc_in);
            else
                stage_attn(s_stage, rg, g.nk, p.att_part + g.l * p.att_layer, p.att_smax, n_split);
            __syncthreads();
            PK_STAMP(ph, kTrStaged);
            if (p.dbg_stage)
                pk_dump_stage(p.dbg_stage + static_cast<size_t>(ph) * p.dbg_stride, s_stage,
                              g.stage == kStNorm ? p.d : (whole ? g.nk * g.V : 0), rg.b, rg.e, g.nk, g.V);
            if constexpr (kA8) {
                if (g.kind != kPhLM) stage_quant_a8(s_stage, whole ? g.nk : rg.e - rg.b);
            }
            if (g.kind == kPhLM) f16_tiles(ring, p.lm, g.nk, rg, rb0, s_stage, s_red);
            else if (kA8)
                w4_tiles_a8(ring, g.wq, g.ws, g.nk, rg, whole, rb0, s_stage, s_red);
            else if (g.kind == kPhD)
                w4_tiles<true>(ring, g.wq, g.ws, g.nk, rg, whole, rb0, s_stage, s_red);
            else
                w4_tiles<false>(ring, g.wq, g.ws, g.nk, rg, whole, rb0, s_stage, s_red);
            PK_STAMP(ph, kTrTiles);
            // publish before issuing the next phase's loads: vmcnt is in
            // order, so waiting for the adds would also wait for the prefetch
            phase_reduce(p, g, s_red, rb0, n_rl, pos, epoch);
            PK_STAMP(ph, kTrSignal);
            if (has_next && !next_after_att) {
                const PhaseDesc gn = phase_desc(p, ph + 1, par, n_split);
                prefetch_phase(ring, p, gn);
            }
        } else {
            if (!ok) break;
            // no tiles here: the work-group still counts as done
            if (g.kind != kPhLM && wave == 0) pk_signal_rep(g.done + (B / kGW) * kCS * kCRep);
            if (has_next && !next_after_att) {
                const PhaseDesc gn = phase_desc(p, ph + 1, par, n_split);
                prefetch_phase(ring, p, gn);
            }
        }
    }

    // clear the other parity's accumulators and counters for the next step
    // (after this work-group's last phase: at the start these 12 MB of stores
    // sat in front of the first dependency wait's loads)
    {
        u32x4 *z = reinterpret_cast<u32x4 *>(p.par[par ^ 1]);
        const size_t n16 = p.par_bytes / 16;
        const u32x4 zero = {0u, 0u, 0u, 0u};
        for (size_t i = static_cast<size_t>(B) * kPkThreads + threadIdx.x; i < n16;
             i += static_cast<size_t>(p.P) * kPkThreads)
            z[i] = zero;
    }
}

}  // namespace w4

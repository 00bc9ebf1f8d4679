/*
 * w4a16.h -- C ABI of the MI355X (gfx950) W4A16 batch-1 decode library.
 *
 * The operations follow the "annotated-llm-runtime" pages:
 *   [TS] "Building a Custom LLM Inference Runtime for Qwen2.5-Coder-7B on
 *        NVIDIA H100 Hopper Architecture" (techsurvey.info),
 *   [SP] "The Architecture of Modern Inference: A Deep Dive into the
 *        Development of the Annotated LLM Runtime for NVIDIA Hopper GPUs"
 *        (snapost.net),
 *   [AI] "How To Build Your Own LLM Runtime From Scratch" (aissential.tech).
 *
 * Conventions for every call:
 *   - No exceptions cross this boundary.  Each call returns a w4_status; on a
 *     failure w4_last_error() (thread-local) holds a readable message.
 *   - "device" pointers are HIP device memory (e.g. a torch CUDA tensor's
 *     data_ptr()), owned by the caller, 16-byte aligned unless stated.
 *     "host" pointers are ordinary CPU memory owned by the caller.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     GPU calls only enqueue work and return; they never allocate.
 *   - fp16 values travel as uint16_t bit patterns (IEEE binary16).
 *   - Argument errors are detected on the host before anything is enqueued;
 *     outputs are then left untouched.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t w4_status;
#define W4_OK       0
#define W4_EINVAL  (-1) /* bad shape or argument                               */
#define W4_EALIGN  (-2) /* a pointer is NULL or not 16-byte aligned            */
#define W4_ERANGE  (-3) /* a code outside [-8, 7] or a non-finite scale        */
#define W4_ESTATE  (-4) /* call out of sequence (position mismatch, no model)  */
#define W4_ENOSPC  (-5) /* the KV page pool or token history is full           */
#define W4_EHIP    (-6) /* the HIP runtime reported an error                   */
#define W4_EFORMAT (-7) /* a weight container failed its checks                */

/* Message of the last failed call on this thread ("" if none). */
const char *w4_last_error(void);

/* Library build identifier (static string). */
const char *w4_version(void);

/* ------------------------------------------------------------------------
 * Packed int4 weights  ([TS] "Technical Specifications and Hardware
 * Alignment": symmetric group-wise INT4, group 128, one fp16 scale per
 * group; [TS] ".nanoqwen File Format": nibbles pre-arranged for the
 * unpacking datapath, here gfx950's 128-bit loads).
 *
 * Logical weights: codes q[N][K] (int8 holding values in [-8, 7]) and scales
 * s[N][K/128] (fp16), W[n][k] = q[n][k] * s[n][k / 128].  K must be a
 * positive multiple of 128.
 *
 * Packed layout (private to the kernels, documented for tests): rows are
 * grouped in blocks of 64 (N is padded up; pad rows have code 0 and scale 0).
 * For row block b, 32-element K chunk c and row r = 64 b + l, the 16 bytes at
 * offset ((b * K/32 + c) * 64 + l) * 16 hold elements k = 32 c .. 32 c + 31 of
 * packed row r as four little-endian 32-bit words; word d holds elements
 * 32 c + 8 d + e, e = 0..7, as nibbles u = q + 8: element 2j in bits
 * [4j, 4j+4), element 2j+1 in bits [16+4j, 16+4j+4).  Scales are stored as
 * packed_s[(b * K/128 + g) * 64 + l] = s[row][g].
 * Packed row r holds logical row row_perm[r] (identity when row_perm is NULL).
 * ------------------------------------------------------------------------ */

/* Bytes of packed codes / packed scales for an N x K matrix (0 if invalid). */
size_t w4_packed_qbytes(int64_t N, int64_t K);
size_t w4_packed_sbytes(int64_t N, int64_t K);

/* Host-side packer.  q, scales, row_perm: host, read-only.  packed_q
 * (w4_packed_qbytes bytes) and packed_s (w4_packed_sbytes bytes): host,
 * written.  group must be 128.  row_perm, if not NULL, is a permutation of
 * [0, N).  Errors: W4_EINVAL (shape, group, bad permutation), W4_ERANGE (a
 * code outside [-8, 7] or a non-finite scale), W4_EALIGN (NULL pointer). */
w4_status pack_int4_weights(const int8_t *q, const uint16_t *scales, int64_t N,
                            int64_t K, int32_t group, const int32_t *row_perm,
                            uint8_t *packed_q, uint16_t *packed_s);

/* fp16 -> int4 quantiser, the step before pack_int4_weights (the pages keep
 * symmetric group-wise int4 weights with one fp16 scale per group of 128
 * but do not give the quantiser).  Per row and group of 128 along K:
 *   scales[n][g] = fp16(max_k |w[n][k]| / 7)   (one rounding of the exact quotient)
 *   q[n][k]      = clamp(round-half-even(w[n][k] / scales[n][g]), -8, 7)
 * and zero codes where the scale rounds to zero.  w: host fp16 [N][K]; q:
 * host int8 [N][K] and scales: host fp16 [N][K/128], written.  group must be
 * 128.  Errors: W4_EINVAL (shape, group), W4_ERANGE (a non-finite weight),
 * W4_EALIGN (NULL pointer). */
w4_status quantize_int4_weights(const uint16_t *w, int64_t N, int64_t K, int32_t group,
                                int8_t *q, uint16_t *scales);

/* Exact inverse of pack_int4_weights (same arguments, data flowing back). */
w4_status unpack_int4_weights(const uint8_t *packed_q, const uint16_t *packed_s,
                              int64_t N, int64_t K, int32_t group,
                              const int32_t *row_perm, int8_t *q,
                              uint16_t *scales);

/* fp16 matrices (the lm_head, [TS] "Technical Specifications…": kept in raw
 * fp16).  Same row blocks of 64; the 16 bytes at ((b * K/8 + c) * 64 + l) * 16
 * hold elements 8c .. 8c+7 of row 64 b + l.  K must be a multiple of 8. */
size_t w4_packed_f16_bytes(int64_t N, int64_t K);
w4_status w4_pack_f16_matrix(const uint16_t *w, int64_t N, int64_t K,
                             uint16_t *packed);

/* ------------------------------------------------------------------------
 * W4A16 GEMV  ([TS] "Engineering Challenges" item 3, the fp16-activation
 * path: int4 weights unpacked on the fly, fp16 activations, no activation
 * quantisation).  y[r] = fp16( sum_k W[r][k] * x[k] ) for packed rows
 * r < N: every 8 consecutive products summed in fp32 as two 4-term chains
 * (each product exact; one fp32 addition per 4 terms may be off by up to one
 * ulp), those 8-term sums and the groups added in fp64.
 *
 *   packed_q, packed_s : device, from pack_int4_weights (any row_perm; y is
 *                        in packed row order)
 *   x                  : device, fp16 [K]
 *   y                  : device, fp16 [N] (written)
 *   workspace          : device, w4_gemv_ws_bytes(N, K) bytes of scratch
 *                        (a mark word, then partial sums of row blocks
 *                        shared by work-groups and their arrival counters).
 *                        It must be all zero before its first use (e.g.
 *                        hipMemset once); the first call sets the mark (the
 *                        first 4 bytes) and every call leaves the rest all
 *                        zero again, whatever the shape, so it can be reused
 *                        across shapes without clearing.  A workspace whose
 *                        mark is neither zero nor the library's (memory that
 *                        was never zeroed) is left untouched and y is filled
 *                        with NaN; corruption after the mark was set is not
 *                        detected.  Calls that share a workspace must be
 *                        ordered on one stream.
 * Errors: W4_EINVAL (N < 1, K not a positive multiple of 128, workspace too
 * small), W4_EALIGN, W4_EHIP (launch failure). */
size_t w4_gemv_ws_bytes(int64_t N, int64_t K);
w4_status w4a16_gemv(const uint8_t *packed_q, const uint16_t *packed_s,
                     const uint16_t *x, uint16_t *y, int64_t N, int64_t K,
                     void *workspace, size_t ws_bytes, void *stream);

/* w4a16_gemv for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernel and result, bit for bit, with the workspace taken from a fixed
 * device array inside the library instead of an argument.  The array holds
 * w4_noalloc_scratch_bytes() bytes (4 MiB) on every GPU the library runs on,
 * until the process ends; shapes whose w4_gemv_ws_bytes(N, K) exceed it are
 * refused with W4_EINVAL (the 7B shapes need at most 576 KiB).  The call
 * allocates nothing (its first call on a device looks up the array's
 * address).  All calls on one GPU share its array and every call leaves it
 * zero again: calls that overlap on one GPU (concurrent streams) race and
 * must be ordered by the caller.  Arguments and errors otherwise as for
 * w4a16_gemv. */
size_t w4_noalloc_scratch_bytes(void);
w4_status w4a16_gemv_noalloc(const uint8_t *packed_q, const uint16_t *packed_s,
                             const uint16_t *x, uint16_t *y, int64_t N, int64_t K,
                             void *stream);

/* ------------------------------------------------------------------------
 * W4A8 GEMV: int8 activations (the pages' integer path, "Path A": [TS]
 * "Engineering Challenges" item 3 and [SP] "Three Critical Engineering
 * Challenges" item 3 compare it with the fp16-activation path on an H100;
 * both weights and activations are integer so the inner products run on
 * integer dot-product instructions, after a separate quantisation step).
 * The pages do not give the activation quantiser; here it is symmetric per
 * group of 128 along K: scale s_g = fp32(max|x| / 127), code
 * c_k = clamp(round-half-even(fp32(x_k / s_g)), -127, 127); an all-zero
 * group has s_g = 0 and zero codes.
 *   y[r] = fp16( sum_g s_w[r][g] * s_g * sum_{k in g} q[r][k] * c_k )
 * with each group's integer sum exact and the groups added in fp64.
 *
 * w4a8_act_bytes(K): size of the quantised-activation buffer (0 for a bad K).
 * w4a8_quantize_act: x device fp16 [K] -> act (device, written).  Layout of
 *   act: bytes [0, K) the codes, each block of 8 elements e0..e7 stored as
 *   the words (e0, e4, e1, e5), (e2, e6, e3, e7); at A = K rounded up to 256
 *   the fp32 scales [K / 128]; at A + (K / 32 rounded up to 256) the int32
 *   sums of each group's codes.  One launch; K a positive multiple of 128.
 * w4a8_gemv: packed_q, packed_s as for w4a16_gemv; act from
 *   w4a8_quantize_act; y device fp16 [N] (packed row order); workspace
 *   w4_gemv_ws_bytes(N, K) bytes with the same contract as for w4a16_gemv
 *   (zero before first use, mark set and the rest left zero).
 * Errors: W4_EINVAL, W4_EALIGN, W4_EHIP. */
size_t w4a8_act_bytes(int64_t K);
w4_status w4a8_quantize_act(const uint16_t *x, int64_t K, void *act, void *stream);
w4_status w4a8_gemv(const uint8_t *packed_q, const uint16_t *packed_s, const void *act,
                    uint16_t *y, int64_t N, int64_t K, void *workspace, size_t ws_bytes,
                    void *stream);

/* The MLP decode block of one token, two launches of the w4a16_gemv kernel:
 * the fused gate+up GEMV with its SwiGLU epilogue, then the down GEMV
 * (SwiGLU MLP of the Qwen2.5-7B decode workload; int4 projections as above).
 *   h = fp16( silu(Wg x) * (Wu x) ),   y = fp16( Wd h )
 *   gu_q, gu_s     : device, the [gate ; up] matrix (2F rows, K = D) packed
 *                    with the W4_PERM_GATE_UP row order (see below)
 *   down_q, down_s : device, Wd (D rows, K = F) packed in identity order
 *   x              : device, fp16 [D];  h : fp16 [F] and y : fp16 [D] (written)
 *   workspace      : device, w4_mlp_ws_bytes(D, F) bytes of scratch, with
 *                    w4a16_gemv's contract (zero before first use)
 * The down GEMV sums as w4a16_gemv does.  The gate+up GEMV, whose input is
 * the block's normalised activation (O(1) entries), chains each group's
 * products in one fp32 accumulator (v_dot2 accumulation: about 40% less VALU
 * work; the accumulator's low bits are cut, which stays within the GEMV
 * tolerance only when outputs are not much smaller than their terms).
 * D and F must be positive multiples of 128.  Errors as for w4a16_gemv. */
size_t w4_mlp_ws_bytes(int64_t D, int64_t F);
w4_status w4a16_mlp(const uint8_t *gu_q, const uint16_t *gu_s, const uint8_t *down_q,
                    const uint16_t *down_s, const uint16_t *x, uint16_t *h, uint16_t *y,
                    int64_t D, int64_t F, void *workspace, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * W4A16 GEMM for prompt prefill (the projections of M prompt tokens at once;
 * the pages time the first token of a 512-token prompt, [SP] "Technical
 * Specifications and Benchmarking Data", performance comparison table, and
 * [AI] "Summary", without describing the prefill).  Matrix cores
 * (MFMA 32x32x16 fp16): within a group of 128 K the integer codes meet the
 * fp16 activations exactly and the products are summed in fp32; each group
 * sum times its fp16 scale is added in fp64; a split of the K groups stores
 * its sum as fp32, and the splits are added in fp64 in split order.
 *   y[m][r] = sum_k x[m][k] * W[r][k]     for m < M, packed rows r < N
 *
 *   packed_q, packed_s : device, from pack_int4_weights (y is in packed row
 *                        order)
 *   x                  : device, fp16 [M][K] row-major, 16-byte aligned
 *   y                  : device, fp32 [M][N] row-major (written)
 *   workspace          : device, w4_gemm_ws_bytes(M, N, K) bytes of scratch
 *                        (split-K partials; no initialisation needed);
 *                        calls sharing it must be ordered on one stream
 * Errors: W4_EINVAL (M outside [1, 2^20], N < 1, K not a positive multiple
 * of 128, workspace too small), W4_EALIGN, W4_EHIP (launch failure). */
size_t w4_gemm_ws_bytes(int64_t M, int64_t N, int64_t K);
w4_status w4a16_gemm(const uint8_t *packed_q, const uint16_t *packed_s,
                     const uint16_t *x, float *y, int64_t M, int64_t N, int64_t K,
                     void *workspace, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Paged decode attention  ([TS] "Technical Specifications…": 16-token pages,
 * one kv-head slice of a page is 4 KiB; [SP] "Three Critical Engineering
 * Challenges" item 1: softmax and weighted-V accumulation over KV pages).
 *
 * out[h] = sum_t softmax_t(scale * q[h] . K[t, h / (n_qh/n_kvh)]) V[t, ...]
 * over the ctx_len cached tokens t; token t lives in physical page
 * page_table[t / 16], slot t % 16.
 *
 *   q           : device, fp16 [n_qh][head_dim]
 *   k_pool,
 *   v_pool      : device, fp16 [n_phys][n_kvh][16][head_dim]
 *   page_table  : device, int32 [n_pages_max]; entries are trusted to be
 *                 valid physical pages of the pools
 *   out         : device, fp16 [n_qh][head_dim] (written)
 *   workspace   : device, w4_attn_ws_bytes(n_qh, n_kvh, n_pages_max) bytes of
 *                 scratch (per-split partials and arrival counters).  It must
 *                 be zero before its first use; each call leaves its counter
 *                 region zero, so reuse (any shape) needs no clearing; calls
 *                 sharing it must be ordered on one stream
 * head_dim must be 128; 1 <= n_kvh <= 256; n_qh a multiple of n_kvh with
 * n_qh / n_kvh in {1, 2, 4, 7, 8}; 1 <= ctx_len <= 16 * n_pages_max.
 * Otherwise W4_EINVAL.  Arithmetic: q.K on the matrix cores (fp16 operands,
 * fp32 sums), softmax in fp32 (base 2), the weights entering the weighted sum
 * of V as an fp16 pair hi + lo (about 22 bits of the fp32 weight), fp32 sums,
 * fp16 output; splits merged in a fixed order (bitwise repeatable). */
size_t w4_attn_ws_bytes(int32_t n_qh, int32_t n_kvh, int32_t n_pages_max);
w4_status paged_attn_decode(const uint16_t *q, const uint16_t *k_pool,
                            const uint16_t *v_pool, const int32_t *page_table,
                            int32_t ctx_len, int32_t n_qh, int32_t n_kvh,
                            int32_t head_dim, int32_t n_pages_max, float scale,
                            uint16_t *out, void *workspace, size_t ws_bytes,
                            void *stream);

/* Causal paged attention of a chunk of prompt tokens (prefill), on matrix
 * cores.  Query m (m < n_tokens) sits at position pos0 + m and attends to the
 * cached positions 0 .. pos0 + m, which include the chunk's own keys:
 *   out[m][h] = sum_{t <= pos0+m} softmax_t(scale * q[m][h] . K[t, kv(h)]) V[t, kv(h)]
 * with kv(h) = h / (n_qh / n_kvh) and token t in physical page
 * page_table[t / 16], slot t % 16 (same pools as paged_attn_decode).
 *   q         : device, fp16 [n_tokens][n_qh][head_dim]
 *   k_pool,
 *   v_pool    : device, fp16 [n_phys][n_kvh][16][head_dim], holding every
 *               position < pos0 + n_tokens
 *   page_table: device, int32; entries for positions < pos0 + n_tokens are
 *               trusted to be valid physical pages
 *   out       : device, fp16 [n_tokens][n_qh][head_dim] (written)
 * head_dim must be 128 and n_qh a multiple of n_kvh; scale > 0.  The
 * softmax weights enter the weighted sum of V rounded to fp16.
 * Errors: W4_EINVAL, W4_EALIGN, W4_EHIP. */
w4_status paged_attn_prefill(const uint16_t *q, const uint16_t *k_pool,
                             const uint16_t *v_pool, const int32_t *page_table,
                             int32_t pos0, int32_t n_tokens, int32_t n_qh,
                             int32_t n_kvh, int32_t head_dim, float scale,
                             uint16_t *out, void *stream);

/* ------------------------------------------------------------------------
 * Decoder model and the graph-captured decode step
 * ([TS] "Engineering Challenges" item 2 and [SP] "Eliminating Host Overhead
 * with CUDA Graphs": the whole step captured once, in a page-boundary and a
 * no-boundary variant picked per step by position modulo 16; [SP]
 * ".nanoqwen Format": no allocation while generating).
 * ------------------------------------------------------------------------ */

typedef struct w4_model w4_model;

typedef struct {
    int32_t d_model;     /* hidden size, multiple of 128                   */
    int32_t d_ff;        /* MLP size, multiple of 128                      */
    int32_t n_layers;
    int32_t n_q_heads;
    int32_t n_kv_heads;  /* n_q_heads / n_kv_heads in {1, 2, 4, 7, 8}      */
    int32_t head_dim;    /* must be 128                                    */
    int32_t vocab;
    int32_t max_pages;   /* KV pool pages per layer; positions < 16*max_pages */
    float eps;           /* RMSNorm epsilon                                */
    double theta;        /* RoPE base                                      */
} w4_model_config;

/* Row orders the model expects its packed projections in (pass the result
 * as row_perm to pack_int4_weights):
 *   W4_PERM_QKV     : N = (n_q_heads + 2 n_kv_heads) * head_dim rows of the
 *                     [q heads | k heads | v heads] matrix; within each head
 *                     packed row 2i holds dim i and 2i+1 holds dim i + 64, so
 *                     the two halves of a rotary pair sit in adjacent lanes.
 *   W4_PERM_GATE_UP : N = 2 d_ff rows of [gate ; up]; packed row 2i holds
 *                     gate row i and 2i+1 holds up row i. */
#define W4_PERM_QKV     0
#define W4_PERM_GATE_UP 1
w4_status w4_model_row_perm(int32_t kind, const w4_model_config *cfg,
                            int32_t *perm /* host, N entries */);

/* Device buffers of a model; all caller-owned and outliving the model.
 * Per-layer entries are host arrays of n_layers device pointers. */
typedef struct {
    const uint8_t *const *qkv_q;      /* packed, W4_PERM_QKV order          */
    const uint16_t *const *qkv_s;
    const uint16_t *const *qkv_bias;  /* fp16 [qkv rows], logical order,
                                         16-byte aligned                    */
    const uint8_t *const *o_q;        /* packed, identity order             */
    const uint16_t *const *o_s;
    const uint8_t *const *gu_q;       /* packed, W4_PERM_GATE_UP order      */
    const uint16_t *const *gu_s;
    const uint8_t *const *down_q;     /* packed, identity order             */
    const uint16_t *const *down_s;
    const uint16_t *const *ln1;       /* fp16 [d_model], 4-byte aligned     */
    const uint16_t *const *ln2;       /* fp16 [d_model], 4-byte aligned     */
    const uint16_t *embed;            /* fp16 [vocab][d_model], row-major   */
    const uint16_t *lnf;              /* fp16 [d_model], 4-byte aligned     */
    const uint16_t *lm_head;          /* w4_pack_f16_matrix of [vocab][d]   */
    uint16_t *k_cache;                /* fp16 [n_layers][max_pages][n_kv][16][128] */
    uint16_t *v_cache;                /* same shape                         */
    int32_t *page_table;              /* int32 [max_pages], written by steps */
    const int32_t *free_list;         /* int32 [max_pages]: physical page for
                                         each successive logical page       */
    int32_t *tokens;                  /* int32 [16*max_pages + 1]: prompt in
                                         [0, n_prompt), generated after     */
    float *logits;                    /* fp32 [vocab], last step's logits   */
} w4_model_buffers;

/* Creates a model: validates cfg and buffers, allocates the library's own
 * workspace (activations, split-K partials, counters, RoPE table) and
 * captures the two step graphs.  This is the only call that allocates. */
w4_status w4_model_create(const w4_model_config *cfg,
                          const w4_model_buffers *buf, w4_model **out);
void w4_model_destroy(w4_model *m);

/* Starts a sequence: position 0, the first n_prompt entries of tokens are
 * the prompt (teacher-forced).  Enqueued on stream. */
w4_status w4_model_reset(w4_model *m, int32_t n_prompt, void *stream);

/* Current host-side position of the model (next position decode_step takes). */
int32_t w4_model_pos(const w4_model *m);

/* One decode step at position pos (must equal the model's position):
 * embeds tokens[pos], runs every layer (RMSNorm, QKV GEMV + bias + RoPE +
 * KV append, paged attention, O GEMV + residual, RMSNorm, gate/up GEMV +
 * SwiGLU, down GEMV + residual), the final norm and the fp16 lm_head, writes
 * logits, and stores the greedy token (lowest index of the maximum) into
 * tokens[pos+1] unless pos+1 < n_prompt.  When pos % 16 == 0 the step first
 * appends free_list[pos/16] to the page table.
 * The step runs as one persistent kernel (dependencies between phases are
 * resolved on the device) or, with W4_MULTI, as one kernel per operation.
 * flags: W4_GRAPH replays the captured graph of the matching variant;
 * W4_EAGER launches the same kernels directly.
 * Errors: W4_ESTATE (pos mismatch), W4_ENOSPC (pos >= 16*max_pages),
 * W4_EINVAL (unknown or conflicting flags), W4_EHIP. */
#define W4_GRAPH 0u   /* replay the captured graph (default)                 */
#define W4_EAGER 1u   /* launch the same kernels directly                     */
#define W4_MULTI 2u   /* with W4_GRAPH/W4_EAGER: the one-kernel-per-operation
                         step (143 launches) instead of the persistent one    */
#define W4_A8    4u   /* with W4_GRAPH/W4_EAGER, not W4_MULTI: the persistent
                         step with int8 activations ([TS] "Engineering
                         Challenges" item 3, Path A): every int4 GEMV input
                         (the normalised residual, the attention output, h)
                         is quantised per group of 128 as w4a8_quantize_act
                         does, and the GEMVs take integer dot products; the
                         lm_head stays fp16.  Its graphs are captured on first
                         use.  W4_EINVAL if a work-group would stage more than
                         32 groups (d_model > 4096).                          */
w4_status decode_step(w4_model *m, int32_t pos, uint32_t flags, void *stream);

/* Prefill of n_tokens (1..512) prompt tokens at positions pos .. pos +
 * n_tokens - 1 (pos must equal the model's position): appends the pages that
 * start in that range, runs every layer over all rows with W4A16 GEMMs
 * (RMSNorm, QKV + bias + RoPE, K/V written into the cache, causal paged
 * attention over positions 0..p, O + residual, RMSNorm, gate/up + SwiGLU,
 * down + residual), then the final norm and the fp16 lm_head on the last row:
 * logits as after a decode step at position pos + n_tokens - 1, and the
 * greedy token stored into tokens[pos + n_tokens] unless pos + n_tokens <
 * n_prompt.  The model's position becomes pos + n_tokens; decode_step
 * continues from there.  Same arithmetic and fp16 storage points as
 * decode_step; the time to first token of a 512-token prompt is one call
 * ([SP] "Technical Specifications and Benchmarking Data").  Launched
 * directly (not graph-captured); uses the model's prefill scratch, so calls
 * on one model must be ordered on one stream.
 * Errors: W4_ESTATE (pos mismatch, no reset), W4_EINVAL (n_tokens outside
 * [1, 512]), W4_ENOSPC (positions beyond the KV pool), W4_EHIP. */
#define W4_PREFILL_MAX 512
w4_status w4_model_prefill(w4_model *m, int32_t pos, int32_t n_tokens, void *stream);

/* Synchronises the device and reports the persistent step's error word:
 * 0 = no error; otherwise the step bailed out and its outputs are invalid:
 * 1000-3999 a dependency wait exceeded its spin limit, 5000 the page-table
 * entry of the step's position lies outside [0, max_pages), 5001 the step's
 * token id lies outside [0, vocab) (checked before anything is read through
 * them). */
w4_status w4_model_status(w4_model *m, int32_t *device_error);

/* Work-groups of the persistent step.  The step's phases hand over through
 * device-memory counters that every work-group waits on, so all of them must
 * be resident at once: the grid is sized from the kernel's occupancy for a
 * device with nothing else running.  decode_step therefore needs the whole
 * device; a kernel running concurrently on another stream can hold CUs the
 * step needs, and its waits then end at their spin limit with a device error.
 * After any device error (w4_model_status non-zero) later steps do nothing
 * (the error word stays set, outputs are stale, the host-side position keeps
 * counting) until w4_model_reset. */
int32_t w4_model_grid(const w4_model *m);

/* ------------------------------------------------------------------------
 * Inspection of the persistent step, for layer-level parity tests.  The
 * step keeps its per-layer intermediates in library-owned device memory:
 *  - acc[par]: int64 accumulators, [n_layers][acc_layer] in fixed point
 *    (value = acc / 2^fix_bits), rows in packed order: the QKV GEMV (without
 *    bias) at acc_q in W4_PERM_QKV row order, the O GEMV at acc_o, the gate/up
 *    GEMV at acc_gu in W4_PERM_GATE_UP order, the down GEMV at acc_d.  A step
 *    fills the block of parity last_parity and clears the other one.
 *  - resid: fp32 [2 n_layers + 1][resid_stride]: the embedding row, then per
 *    layer the residual stream after the O projection and after the down
 *    projection.
 *  - att_part: fp32 attention chunk partials, att_layer_floats per layer; per
 *    query head att_smax chunks of 132 floats: running max of the scores in
 *    log2 units, sum of exponentials, 2 unused, 128 weighted sums of V.  Chunk
 *    c covers pages [c, c+1) * att_pages_per_chunk.
 * Pointers stay valid until w4_model_destroy.  Synchronises the device.
 * Errors: W4_EINVAL, W4_EHIP. */
typedef struct {
    const void *acc[2];
    int64_t acc_layer;
    int32_t acc_q, acc_o, acc_gu, acc_d;
    int32_t fix_bits;
    int32_t last_parity;
    const float *resid;
    int64_t resid_stride;
    const float *att_part;
    int64_t att_layer_floats;
    int32_t att_smax, att_pages_per_chunk;
    int32_t stage_stride;
    int32_t reserved;
} w4_debug_layout;
w4_status w4_model_debug_layout(w4_model *m, w4_debug_layout *out);

/* Staged-input dump for the same tests: with buf set (device memory, fp16,
 * w4_model_stage_dump_elems(m) elements, caller-owned), every later
 * persistent step also writes the fp16 input each GEMV phase read, phase ph
 * at buf + ph * stage_stride: per layer (ph = 4 l + k) the normalised input of
 * the QKV GEMV (k = 0, d elements), the attention output entering the O GEMV
 * (k = 1, n_q_heads * 128), the normalised input of the gate/up GEMV (k = 2,
 * d) and the SwiGLU output entering the down GEMV (k = 3, d_ff); then the
 * final normalised state entering the lm_head (ph = 4 n_layers, d).  NULL
 * turns the dump off (the default).  Synchronises the device.
 * Errors: W4_EINVAL, W4_EALIGN, W4_EHIP. */
size_t w4_model_stage_dump_elems(const w4_model *m);
w4_status w4_model_set_stage_dump(w4_model *m, uint16_t *buf);

/* Number of kernel launches one step of the variant selected by flags
 * (W4_MULTI or not) makes, not counting the page append that steps at a page
 * boundary add (for the launch-count report). */
int32_t w4_model_launches_per_step(const w4_model *m, uint32_t flags);

/* Measurement hook: enqueues `reps` launches of one of the step's kernels,
 * with the step's launch geometry, cycling over the layers' weights (so
 * consecutive launches stream distinct weights from HBM).  The launches read
 * and overwrite the model's activation scratch: call w4_model_reset before
 * the next decode_step.  kind: W4_KERNEL_GATE_UP (gate+up GEMV + SwiGLU),
 * W4_KERNEL_DOWN (down GEMV + residual), W4_KERNEL_O (O GEMV + residual),
 * W4_KERNEL_LM_HEAD (fp16 lm_head GEMV + argmax).  Errors: W4_EINVAL. */
#define W4_KERNEL_GATE_UP 0
#define W4_KERNEL_DOWN    1
#define W4_KERNEL_O       2
#define W4_KERNEL_LM_HEAD 3
w4_status w4_model_kernel_replay(w4_model *m, int32_t kind, int32_t reps, void *stream);

/* ------------------------------------------------------------------------
 * Weight container: a memory-mappable file of packed tensors ([TS] ".nanoqwen
 * File Format and Safety Protocols" and [SP] "Data Integrity and
 * Serialization": a fixed 256-byte header opening with an 8-byte magic
 * string, checked first so a wrong file is refused, then weights stored in
 * the kernels' packed layout; here the gfx950 layout, with its own magic
 * "W4GFX950").  Layout: the 256-byte header (magic, version 1, sizes, tensor
 * count, table offset 256, file size, FNV-1a 64 checksum of the table, the
 * model config), a table of 96-byte entries (name up to 47 bytes, kind, row
 * order, rows, cols, offset, bytes), then each tensor at a 4096-byte aligned
 * offset.  Host-side only; the mapped bytes are uploaded by the caller.
 * ------------------------------------------------------------------------ */
#define W4C_INT4_CODES  0   /* pack_int4_weights codes, rows x cols logical  */
#define W4C_INT4_SCALES 1   /* pack_int4_weights scales                      */
#define W4C_F16         2   /* raw fp16 [rows][cols]                         */
#define W4C_F16_ROWS    3   /* w4_pack_f16_matrix rows                       */
typedef struct {
    const char *name;    /* NUL-terminated, at most 47 bytes                  */
    int32_t kind;        /* W4C_*                                             */
    int32_t row_order;   /* informational: W4_PERM_* + 1, or 0 for identity   */
    int64_t rows, cols;
    const void *data;    /* host bytes (write) / inside the mapping (read)    */
    size_t bytes;        /* must equal what kind, rows and cols imply         */
} w4c_tensor;
typedef struct w4c_file w4c_file;

/* Writes the container (tensors in the given order).  Errors: W4_EINVAL. */
w4_status w4c_write(const char *path, const w4_model_config *cfg, int32_t n_tensors,
                    const w4c_tensor *tensors);
/* Maps a container read-only after checking, in order: size and magic (read
 * before mapping), version, header and entry sizes, file size, table bounds
 * and checksum, and every entry (name, kind, byte count for its shape,
 * 4096-byte alignment, bounds, order).  Errors: W4_EFORMAT (a check failed;
 * the message names it), W4_EINVAL (cannot open or map). */
w4_status w4c_open(const char *path, w4c_file **out);
int32_t w4c_count(const w4c_file *f);
w4_status w4c_config(const w4c_file *f, w4_model_config *cfg);
/* Tensor i, or the tensor with this name; data points into the mapping and
 * stays valid until w4c_close. */
w4_status w4c_tensor_at(const w4c_file *f, int32_t i, w4c_tensor *t);
w4_status w4c_find(const w4c_file *f, const char *name, w4c_tensor *t);
void w4c_close(w4c_file *f);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */

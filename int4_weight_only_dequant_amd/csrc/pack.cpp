// Host-side packers and error reporting of the W4A16 library.
//
// The int4 layout follows the pages' idea of pre-arranging nibbles for the
// unpacking datapath (".nanoqwen File Format" section of "Building a Custom
// LLM Inference Runtime for Qwen2.5-Coder-7B on NVIDIA H100 Hopper
// Architecture"), re-derived for gfx950: one 16-byte load per lane covers 32
// consecutive K elements of that lane's row, and inside each 32-bit word the
// even elements sit in the low half-word and the odd ones in the high
// half-word, so that masking one nibble per half-word and OR-ing the fp16
// exponent pattern 0x6400 yields a pair of fp16 values (1024 + u) ready for a
// two-wide fp16 dot product with two consecutive activations.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "w4_common.hpp"

namespace w4 {

static thread_local char g_err[512] = "";

w4_status fail(w4_status code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_err[0] = 0; }

static bool f16_finite(uint16_t b) { return ((b >> 10) & 0x1F) != 0x1F; }

static int64_t row_blocks(int64_t n) { return (n + kRows - 1) / kRows; }

static w4_status check_perm(const int32_t *perm, int64_t n) {
    if (!perm) return W4_OK;
    std::vector<uint8_t> seen(static_cast<size_t>(n), 0);
    for (int64_t i = 0; i < n; ++i) {
        int32_t p = perm[i];
        if (p < 0 || p >= n || seen[p]) return fail(W4_EINVAL, "row_perm is not a permutation of [0, %lld)", (long long)n);
        seen[p] = 1;
    }
    return W4_OK;
}

static w4_status check_shape(int64_t n, int64_t k, int32_t group) {
    if (group != kGroup) return fail(W4_EINVAL, "group must be %d (got %d)", kGroup, group);
    if (n < 1 || k < kGroup || k % kGroup) return fail(W4_EINVAL, "bad shape N=%lld K=%lld (K must be a positive multiple of 128)", (long long)n, (long long)k);
    if (n > (int64_t(1) << 31) || k > (int64_t(1) << 30)) return fail(W4_EINVAL, "shape too large");
    return W4_OK;
}

// Byte offset of the 16-byte lane slot (row block b, chunk c, lane l).
static inline size_t slot_offset(int64_t b, int64_t c, int64_t l, int64_t n_chunks) {
    return static_cast<size_t>(((b * n_chunks + c) * kRows + l) * 16);
}

// Bit position of element e (0..7) inside its 32-bit word.
static inline int nibble_shift(int e) { return (e & 1) ? 16 + 4 * (e >> 1) : 4 * (e >> 1); }

}  // namespace w4

using namespace w4;

extern "C" {

const char *w4_last_error(void) { return g_err; }

const char *w4_version(void) { return "w4a16-gfx950 0.1"; }

size_t w4_packed_qbytes(int64_t N, int64_t K) {
    if (N < 1 || K < kGroup || K % kGroup) return 0;
    return static_cast<size_t>(row_blocks(N) * kRows * (K / 2));
}

size_t w4_packed_sbytes(int64_t N, int64_t K) {
    if (N < 1 || K < kGroup || K % kGroup) return 0;
    return static_cast<size_t>(row_blocks(N) * kRows * (K / kGroup) * 2);
}

w4_status pack_int4_weights(const int8_t *q, const uint16_t *scales, int64_t N, int64_t K,
                            int32_t group, const int32_t *row_perm, uint8_t *packed_q,
                            uint16_t *packed_s) {
    clear_error();
    if (!q || !scales || !packed_q || !packed_s) return fail(W4_EALIGN, "NULL pointer");
    w4_status st = check_shape(N, K, group);
    if (st) return st;
    if ((st = check_perm(row_perm, N))) return st;
    const int64_t n_chunks = K / kChunk, n_groups = K / kGroup, nb = row_blocks(N);
    // validate everything before writing anything
    for (int64_t i = 0; i < N * K; ++i)
        if (q[i] < -8 || q[i] > 7) return fail(W4_ERANGE, "code %d at flat index %lld outside [-8, 7]", q[i], (long long)i);
    for (int64_t i = 0; i < N * n_groups; ++i)
        if (!f16_finite(scales[i])) return fail(W4_ERANGE, "non-finite scale at flat index %lld", (long long)i);

    for (int64_t b = 0; b < nb; ++b) {
        for (int64_t l = 0; l < kRows; ++l) {
            const int64_t r = b * kRows + l;
            const int64_t src = r < N ? (row_perm ? row_perm[r] : r) : -1;
            const int8_t *qr = src >= 0 ? q + src * K : nullptr;
            for (int64_t c = 0; c < n_chunks; ++c) {
                uint32_t words[4];
                for (int d = 0; d < 4; ++d) {
                    uint32_t w = 0;
                    for (int e = 0; e < 8; ++e) {
                        const int64_t k = c * kChunk + d * 8 + e;
                        const uint32_t u = static_cast<uint32_t>((qr ? qr[k] : 0) + 8);
                        w |= u << nibble_shift(e);
                    }
                    words[d] = w;
                }
                memcpy(packed_q + slot_offset(b, c, l, n_chunks), words, 16);
            }
            for (int64_t g = 0; g < n_groups; ++g)
                packed_s[(b * n_groups + g) * kRows + l] = src >= 0 ? scales[src * n_groups + g] : 0;
        }
    }
    return W4_OK;
}

w4_status unpack_int4_weights(const uint8_t *packed_q, const uint16_t *packed_s, int64_t N,
                              int64_t K, int32_t group, const int32_t *row_perm, int8_t *q,
                              uint16_t *scales) {
    clear_error();
    if (!q || !scales || !packed_q || !packed_s) return fail(W4_EALIGN, "NULL pointer");
    w4_status st = check_shape(N, K, group);
    if (st) return st;
    if ((st = check_perm(row_perm, N))) return st;
    const int64_t n_chunks = K / kChunk, n_groups = K / kGroup;
    for (int64_t r = 0; r < N; ++r) {
        const int64_t b = r / kRows, l = r % kRows;
        const int64_t dst = row_perm ? row_perm[r] : r;
        for (int64_t c = 0; c < n_chunks; ++c) {
            uint32_t words[4];
            memcpy(words, packed_q + slot_offset(b, c, l, n_chunks), 16);
            for (int d = 0; d < 4; ++d)
                for (int e = 0; e < 8; ++e)
                    q[dst * K + c * kChunk + d * 8 + e] =
                        static_cast<int8_t>(static_cast<int>((words[d] >> nibble_shift(e)) & 0xF) - 8);
        }
        for (int64_t g = 0; g < n_groups; ++g)
            scales[dst * n_groups + g] = packed_s[(b * n_groups + g) * kRows + l];
    }
    return W4_OK;
}

size_t w4_packed_f16_bytes(int64_t N, int64_t K) {
    if (N < 1 || K < 8 || K % 8) return 0;
    return static_cast<size_t>(row_blocks(N) * kRows * K * 2);
}

w4_status w4_pack_f16_matrix(const uint16_t *w, int64_t N, int64_t K, uint16_t *packed) {
    clear_error();
    if (!w || !packed) return fail(W4_EALIGN, "NULL pointer");
    if (N < 1 || K < 8 || K % 8) return fail(W4_EINVAL, "bad shape N=%lld K=%lld (K must be a multiple of 8)", (long long)N, (long long)K);
    const int64_t nb = row_blocks(N), n_chunks = K / 8;
    for (int64_t b = 0; b < nb; ++b)
        for (int64_t c = 0; c < n_chunks; ++c)
            for (int64_t l = 0; l < kRows; ++l) {
                const int64_t r = b * kRows + l;
                uint16_t *dst = packed + ((b * n_chunks + c) * kRows + l) * 8;
                if (r < N) memcpy(dst, w + r * K + c * 8, 16);
                else memset(dst, 0, 16);
            }
    return W4_OK;
}

// fp16 -> int4 quantiser: scale = fp16(max|w| / 7) (the fp64 quotient of two
// values with at most 11 significant bits is rounded once more to fp16; the
// exact quotient's binary expansion repeats with period 3, so it is never
// within fp64 rounding of an fp16 tie and the two roundings equal one),
// code = clamp(round-half-even(w / scale), -8, 7), exact in fp64 (a tie of
// w / scale cannot be created or lost by the fp64 quotient either).
static double f16_value(uint16_t b) {
    const int e = (b >> 10) & 0x1F, m = b & 0x3FF;
    const double v = e ? ldexp(1024.0 + m, e - 25) : ldexp(static_cast<double>(m), -24);
    return (b & 0x8000) ? -v : v;
}

w4_status quantize_int4_weights(const uint16_t *w, int64_t N, int64_t K, int32_t group, int8_t *q,
                                uint16_t *scales) {
    clear_error();
    if (!w || !q || !scales) return fail(W4_EALIGN, "NULL pointer");
    const w4_status st = check_shape(N, K, group);
    if (st != W4_OK) return st;
    const int64_t ng = K / kGroup;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < ng; ++g) {
            const uint16_t *wg = w + n * K + g * kGroup;
            double amax = 0.0;
            for (int i = 0; i < kGroup; ++i) {
                if (!f16_finite(wg[i])) return fail(W4_ERANGE, "non-finite weight at (%lld, %lld)", (long long)n, (long long)(g * kGroup + i));
                amax = fmax(amax, fabs(f16_value(wg[i])));
            }
            const _Float16 s16 = static_cast<_Float16>(amax / 7.0);
            uint16_t sbits;
            memcpy(&sbits, &s16, 2);
            scales[n * ng + g] = sbits;
            const double sv = static_cast<double>(s16);
            int8_t *qg = q + n * K + g * kGroup;
            for (int i = 0; i < kGroup; ++i) {
                double c = sv > 0.0 ? nearbyint(f16_value(wg[i]) / sv) : 0.0;   // ties to even
                c = c < -8.0 ? -8.0 : (c > 7.0 ? 7.0 : c);
                qg[i] = static_cast<int8_t>(c);
            }
        }
    }
    return W4_OK;
}

w4_status w4_model_row_perm(int32_t kind, const w4_model_config *cfg, int32_t *perm) {
    clear_error();
    if (!cfg || !perm) return fail(W4_EALIGN, "NULL pointer");
    if (cfg->head_dim != kHeadDim) return fail(W4_EINVAL, "head_dim must be 128");
    if (kind == W4_PERM_QKV) {
        const int64_t heads = int64_t(cfg->n_q_heads) + 2 * int64_t(cfg->n_kv_heads);
        for (int64_t h = 0; h < heads; ++h)
            for (int i = 0; i < kHeadDim / 2; ++i) {
                perm[h * kHeadDim + 2 * i] = static_cast<int32_t>(h * kHeadDim + i);
                perm[h * kHeadDim + 2 * i + 1] = static_cast<int32_t>(h * kHeadDim + i + kHeadDim / 2);
            }
        return W4_OK;
    }
    if (kind == W4_PERM_GATE_UP) {
        for (int64_t i = 0; i < cfg->d_ff; ++i) {
            perm[2 * i] = static_cast<int32_t>(i);
            perm[2 * i + 1] = static_cast<int32_t>(cfg->d_ff + i);
        }
        return W4_OK;
    }
    return fail(W4_EINVAL, "unknown permutation kind %d", kind);
}

}  // extern "C"

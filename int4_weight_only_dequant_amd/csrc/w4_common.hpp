// Shared definitions of the gfx950 W4A16 decode library (host + device).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "w4a16.h"

namespace w4 {

constexpr int kRows = 64;       // rows per row block: one per lane of a wave
constexpr int kGroup = 128;     // K elements sharing one fp16 scale
constexpr int kChunk = 32;      // K elements per 16-byte lane load of codes
constexpr int kPage = 16;       // tokens per KV page
constexpr int kHeadDim = 128;
constexpr int kThreads = 256;   // work-group size of every kernel (4 waves)

// Records a formatted message as this thread's last error and returns code.
w4_status fail(w4_status code, const char *fmt, ...);
void clear_error();

inline bool aligned16(const void *p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace w4

#define W4_HIP(expr)                                                                \
    do {                                                                            \
        hipError_t e_ = (expr);                                                     \
        if (e_ != hipSuccess)                                                       \
            return ::w4::fail(W4_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

#define W4_CHECK(cond, code, ...)                  \
    do {                                           \
        if (!(cond)) return ::w4::fail(code, __VA_ARGS__); \
    } while (0)

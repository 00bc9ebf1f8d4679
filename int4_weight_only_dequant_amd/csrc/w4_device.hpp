// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include "w4_common.hpp"

namespace w4 {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }

// Read-only-for-the-kernel view of global memory (AMDGPU constant address
// space): wave-uniform loads through it become scalar (s_load) reads.
typedef __attribute__((address_space(4))) const uint32_t *const_u32_ptr;
__device__ __forceinline__ const_u32_ptr as_const(const uint32_t *p) {
    return (const_u32_ptr)(p);
}

// A value the compiler must keep in a VGPR: lets three-operand VALU ops
// (v_and_or_b32) take their constants from registers, since gfx9 VOP3
// encodings cannot carry a literal.
__device__ __forceinline__ uint32_t vreg_const(uint32_t c) {
    uint32_t r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
    return r;
}

__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
}

__device__ __forceinline__ float f16_to_f32(uint16_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

__device__ __forceinline__ uint16_t f32_to_f16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// float64 -> binary16 with a single round-to-nearest-even: round to fp32 with
// round-to-odd first (fp32 keeps more than two extra bits), then RNE to fp16.
__device__ __forceinline__ uint16_t f64_to_f16(double d) {
    float f = static_cast<float>(d);
    uint32_t u = __float_as_uint(f);
    if (static_cast<double>(f) != d && (u & 0x7F800000u) != 0x7F800000u) {
        if (fabs(static_cast<double>(f)) > fabs(d)) u -= 1;  // truncate toward zero
        u |= 1u;                                            // sticky bit
    }
    return f32_to_f16(__uint_as_float(u));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
__device__ __forceinline__ float row16_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)); // quad_perm [1,0,3,2]
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)); // quad_perm [2,3,0,1]
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)); // row_half_mirror
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)); // row_mirror
    return v;
}

__device__ __forceinline__ double shfl_xor1(double v) {
    // exchange with the neighbouring lane (quad_perm [1,0,3,2]) on both halves
    uint64_t b = __builtin_bit_cast(uint64_t, v);
    int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(b), 0xB1, 0xF, 0xF, false);
    int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), 0xB1, 0xF, 0xF, false);
    return __builtin_bit_cast(double, (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo));
}

// Device-scope coherent accesses for data exchanged between work-groups that
// may run on different XCDs (each XCD has its own L2).
template <class T>
__device__ __forceinline__ void store_agent(T *p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T load_agent(const T *p) {
    return __hip_atomic_load(const_cast<T *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Last-arriver election: every work-group of a reduction calls this once
// (from one full wave) after publishing its partial; returns true in exactly
// one of them, which then sees all partials.  The winner resets the counter.
//
// Partials are written with store_agent and read with load_agent: device-
// scope accesses (sc1) that complete at the device's coherence point, past
// the per-XCD L2s.  So a work-group fence (wait until this wave's stores are
// acknowledged, no compiler reordering) is enough before the arrival atomic;
// an agent-scope fence would also write back and invalidate the whole L2,
// which costs microseconds per work-group.  Partials stored by other waves of
// the work-group are covered by the __syncthreads() the callers place before
// this call (its release waits for their stores).
__device__ __forceinline__ bool arrive_last(unsigned *counter, unsigned n_arrivals) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    unsigned old = 0;
    if ((threadIdx.x & 63) == 0) old = atomicAdd(counter, 1u);
    old = __builtin_amdgcn_readfirstlane(old);
    const bool last = old == n_arrivals - 1;
    if (last) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        if ((threadIdx.x & 63) == 0) store_agent(counter, 0u);
    }
    return last;
}

}  // namespace w4

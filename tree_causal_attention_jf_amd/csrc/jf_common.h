// Device-side helpers shared by the gfx950 kernels of libjf_tree.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "jf_tree.h"

namespace jf {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kAncWords = 4;
constexpr int kPage = JF_PAGE_SIZE;
constexpr int kNumXcd = 8;           // MI355X: 8 XCDs, workgroups dealt round-robin

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Two floats -> packed bf16x2 (round to nearest even; one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Workgroup id -> logical id such that each XCD receives one contiguous range
// of logical ids (hardware deals workgroup x to XCD x % 8).
__device__ __forceinline__ int xcd_remap(int x, int total) {
    const int q = total / kNumXcd, rem = total % kNumXcd;
    const int xcd = x % kNumXcd, slot = x / kNumXcd;
    return xcd * q + (xcd < rem ? xcd : rem) + slot;
}

// Release this workgroup's prior global writes and bump an agent-scope
// counter; returns the old value. Every thread must have issued a
// __threadfence() after its own writes and the workgroup must be at a barrier.
__device__ __forceinline__ int arrive(int* counter) {
    return __hip_atomic_fetch_add(counter, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void reset_counter(int* counter) {
    __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace jf

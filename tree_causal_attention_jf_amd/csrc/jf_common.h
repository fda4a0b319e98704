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

// Every workspace starts with a counter region of this fixed size, whatever the
// shape of the call: counters are zero before and after every call, and
// everything past them is scratch each call writes before it reads. So one
// workspace can serve calls of any shape, one at a time.
constexpr int kCounterBytes = JF_WORKSPACE_COUNTER_BYTES;
constexpr int kMaxCounters = kCounterBytes / 4;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Two floats -> packed bf16x2 (round to nearest even; one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// max(a, b, c) in one v_max3_f32, without the NaN-quieting copies the compiler
// adds around fmaxf. A quiet NaN input is ignored; a signalling NaN makes the
// result NaN, so callers whose inputs may hold NaN check the result.
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// bf16 pair in one dword -> the two values as fp32 (low half first)
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Largest of the EPV values in a 16-byte vector, folded into m with v_max3
// (a quiet NaN is ignored; a signalling NaN makes the result NaN).
template <typename T>
__device__ __forceinline__ float vec_max(const u32x4 r, float m) {
    if constexpr (sizeof(T) == 2) {
        const float a = max3f(bf_hi(r[0]), bf_hi(r[1]), bf_hi(r[2]));
        const float c = max3f(bf_hi(r[3]), bf_lo(r[0]), bf_lo(r[1]));
        return max3f(max3f(bf_lo(r[2]), bf_lo(r[3]), a), c, m);
    } else {
        return max3f(max3f(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[2])),
                     __uint_as_float(r[3]), m);
    }
}

// Value e (0 .. EPV-1, in index order) of a 16-byte vector.
template <typename T>
__device__ __forceinline__ float vec_val(const u32x4 r, int e) {
    if constexpr (sizeof(T) == 2) return (e & 1) ? bf_hi(r[e >> 1]) : bf_lo(r[e >> 1]);
    else return __uint_as_float(r[e]);
}

// Wave-wide max / min without LDS: DPP steps inside each row of 16 lanes (quad
// permutations, then the half-row and row mirrors), then the four row results
// read with readlane. The result is the same in every lane (scalar).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
constexpr int kDppQuad1032 = 0xb1, kDppQuad2301 = 0x4e, kDppRowHalfMirror = 0x141, kDppRowMirror = 0x140;

__device__ __forceinline__ float wave_max_f32(float v) {
    v = fmaxf(v, __uint_as_float(dpp_u32<kDppQuad1032>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_u32<kDppQuad2301>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_u32<kDppRowHalfMirror>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_u32<kDppRowMirror>(__float_as_uint(v))));
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

__device__ __forceinline__ int wave_min_i32(int v) {
    v = min(v, (int)dpp_u32<kDppQuad1032>((uint32_t)v));
    v = min(v, (int)dpp_u32<kDppQuad2301>((uint32_t)v));
    v = min(v, (int)dpp_u32<kDppRowHalfMirror>((uint32_t)v));
    v = min(v, (int)dpp_u32<kDppRowMirror>((uint32_t)v));
    return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Ancestor-or-self sets of one tree (N <= 256 nodes, 256 bits each) from its
// parent array, in LDS, by pointer doubling: after round k node i holds every
// node within distance < 2^k above it and a pointer to its 2^k-th ancestor, so
// at most 8 rounds cover any tree. A parent entry that breaks the tree rules
// (parent[0] != -1, or parent[i] outside [0, i)) is read as -1, a root, as
// jf_build_ancestor_mask reads it. One thread per node: the workgroup has at
// least N threads, every thread calls this (it holds barriers), and thread i
// passes parent[i] (loaded early by the caller, so its latency hides behind
// other loads; any value for i >= N). Returns the LDS array of sets, complete
// for nodes < N when the call returns.
__device__ __forceinline__ const uint64_t (*tree_sets_lds(int p, int N))[kAncWords] {
    __shared__ uint64_t s_set[JF_MAX_NODES][kAncWords];
    __shared__ int16_t s_up[JF_MAX_NODES];
    const int i = threadIdx.x;
    const bool mine = i < N;
    if (mine) {
        if (!((i == 0) ? (p == -1) : (p >= 0 && p < i))) p = -1;
        #pragma unroll
        for (int w = 0; w < kAncWords; ++w) s_set[i][w] = (w == (i >> 6)) ? (1ull << (i & 63)) : 0ull;
        s_up[i] = (int16_t)p;
    }
    __syncthreads();
    for (int round = 0; round < 8; ++round) {
        uint64_t v[kAncWords];
        int jj = -1;
        if (mine) {
            const int j = s_up[i];
            #pragma unroll
            for (int w = 0; w < kAncWords; ++w) v[w] = s_set[i][w];
            if (j >= 0) {
                #pragma unroll
                for (int w = 0; w < kAncWords; ++w) v[w] |= s_set[j][w];
                jj = s_up[j];
            }
        }
        __syncthreads();                                   // every read of this round before any write
        if (mine) {
            #pragma unroll
            for (int w = 0; w < kAncWords; ++w) s_set[i][w] = v[w];
            s_up[i] = (int16_t)jj;
        }
        if (!__syncthreads_or(mine && jj >= 0)) break;
    }
    return s_set;
}

// The same for trees of at most 64 nodes, inside one wave: lane l < N ends with
// node l's set (bits 0..63), by pointer doubling across the lanes with
// shuffles, so no LDS and no barrier; every wave may run it on its own. p is
// parent[lane] (any value for lanes >= N). At most 7 rounds: a pointer only
// moves up, and its distance doubles each round.
__device__ __forceinline__ uint64_t tree_set_wave(int p, int N) {
    const int l = threadIdx.x & 63;
    const bool mine = l < N;
    if (!mine || !((l == 0) ? (p == -1) : (p >= 0 && p < l))) p = -1;
    uint64_t set = mine ? (1ull << l) : 0ull;
    int up = p;
    for (int round = 0; round < 7 && __any(up >= 0); ++round) {
        const int j = up >= 0 ? up : l;
        const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)set, j);
        const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(set >> 32), j);
        const int uj = __shfl(up, j);
        if (up >= 0) {
            set |= ((uint64_t)hi << 32) | lo;
            up = uj;
        }
    }
    return set;
}

// Workgroup id -> logical id such that each XCD receives one contiguous range
// of logical ids (hardware deals workgroup x to XCD x % 8).
__device__ __forceinline__ int xcd_remap(int x, int total) {
    const int q = total / kNumXcd, rem = total % kNumXcd;
    const int xcd = x % kNumXcd, slot = x / kNumXcd;
    return xcd * q + (xcd < rem ? xcd : rem) + slot;
}

// Cross-workgroup hand-off (split merge, argmax merge, acceptance walk).
//
// MI355X has one L2 per XCD and they are not coherent with each other, so a
// result read by a workgroup on another XCD has to be pushed past the writer's
// L2 and must not be served from a stale line of the reader's.
//
// Bulk results (attention partials, tens of KB per workgroup):
//   writer: device-scope (write-through) stores st16 / st8, wait_own_stores()
//           in every wave, barrier, then ONE thread bumps the counter with
//           arrive(); no cache-wide write-back is needed, and many workgroups
//           publishing at once do not serialize on one;
//   reader: the thread that saw the last arrival calls acquire_agent()
//           (invalidates this CU's L1 and this XCD's L2), and only then
//           resets the counter (the fence waits for every store issued before
//           it, a full round trip for a write-through one), tells the
//           workgroup through LDS and a barrier, and the workgroup then loads
//           normally.
// Small results (8-byte argmax keys) are written and read with agent-scope
// atomics, which bypass the non-coherent caches, and counted with arrive().
__device__ __forceinline__ void wait_own_stores() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ int arrive(int* counter) {
    return __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

__device__ __forceinline__ void reset_counter(int* counter) {
    __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Raw buffer over `bytes` bytes at `base` (out-of-range accesses read 0 and drop writes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

constexpr int kDeviceScope = 16;   // buffer-instruction cache policy sc1: write through to device scope

__device__ __forceinline__ void st16(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kDeviceScope);
}

__device__ __forceinline__ f32x4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ void st8(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kDeviceScope);
}

__device__ __forceinline__ u32x2 ld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}

}  // namespace jf

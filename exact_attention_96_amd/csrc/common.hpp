// Shared device helpers for the attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kLog2e = 1.442695040888963407360f;

// Workgroups are dealt to the 8 XCDs of the chip round-robin by their linear
// id.  Re-number them so that each XCD receives one contiguous range of
// logical tiles: the query tiles of one head then run on one XCD and share
// its L2 copy of that head's K and V.  A bijection on [0, total).
__device__ __forceinline__ int xcd_contiguous(int linear, int total) {
    const int per = total >> 3, rem = total & 7;
    const int xcd = linear & 7, slot = linear >> 3;
    const int first = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
    return first + slot;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace attn

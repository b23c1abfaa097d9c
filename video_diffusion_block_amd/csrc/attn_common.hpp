// Types and small device helpers shared by the attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace bsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16-byte raw chunk as a native vector (HIP's uint4 class defeats register
// promotion of arrays of it).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T>
__device__ inline float to_f32(T v) {
  return (float)v;
}

template <typename T>
__device__ inline T from_f32(float v) {
  return (T)v;
}

// D(32x32 f32) += A(32x16 bf16) * B(16x32 bf16) on the matrix cores.
// Operand layout (64 lanes, l32 = lane % 32, hi = lane / 32):
//   A: lane holds A[l32][8*hi .. 8*hi+7]; B: lane holds B[8*hi .. 8*hi+7][l32];
//   D: lane holds D[8*(r/4) + 4*hi + r%4][l32] in element r (0..15).
__device__ inline f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace bsa

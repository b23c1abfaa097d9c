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

// Pad keys of a partial key block get the score -2^30 from the matrix unit
// instead of a per-score mask (forward and dQ kernels, whose score tiles are
// S^T, keys by queries): the S^T accumulators start from one product
// whose A operand holds, in k-column 0 of key row l32, 0 for a real key and
// -2^30 for a pad key, and whose B operand holds 1 in k-row 0 of every query
// column (pad_bias_b). Real keys start from an exact 0, so their scores are
// bit-identical to a zero start; a pad key's score is -2^30 (about -1.4e8 in
// the exponent's units once scaled), whose exponential is exactly 0 whatever
// is subtracted from it (a real key's running maximum in the forward, the
// row's lse in the dQ kernel). Per 32-key tile this is one product and two
// instructions to form the operand, in place of three instructions per score.
__device__ inline bf16x8 pad_bias_a(uint32_t word, int l32, int hi) {
  const bool pad = hi == 0 && !((word >> l32) & 1u);
  const u32x4 v = {pad ? 0xCE80u : 0u, 0u, 0u, 0u};  // element 0: bf16 -2^30 or 0
  return __builtin_bit_cast(bf16x8, v);
}
__device__ inline bf16x8 pad_bias_b(int hi) {
  const u32x4 v = {hi == 0 ? 0x3F80u : 0u, 0u, 0u, 0u};  // element 0: bf16 1.0 or 0
  return __builtin_bit_cast(bf16x8, v);
}

// Work item of a workgroup of a 2-D grid (x fastest), in an L2-aware order:
// workgroups are handed to the 8 XCDs round-robin (dispatch b runs on XCD
// b % 8, each XCD with its own L2), so inside every window of 256 dispatches
// XCD x takes 32 consecutive items. Neighbouring blocks of one head, whose
// block lists overlap, then share an L2, and the window keeps all XCDs on
// nearby items. A bijection on [0, T); the last partial window is in order.
__device__ inline void xcd_item(int& x, int& y) {
  const int T = gridDim.x * gridDim.y;
  const int b = blockIdx.x + gridDim.x * blockIdx.y;
  int item = b;
  if (b < (T / 256) * 256) item = (b & ~255) + (b & 7) * 32 + ((b >> 3) & 31);
  x = item % gridDim.x;
  y = item / gridDim.x;
}

// ---- direct global -> LDS loads through a buffer resource -------------------
// The buffer form (buffer_load_dwordx4 ... lds) is counted by vmcnt only; the
// flat/global form is also treated by the compiler as a possible LDS access of
// unknown order, which turns every later LDS-read wait into a full wait.
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

extern "C" __device__ void bsa_raw_buffer_load_lds(i32x4 rsrc, lds_void* lds, int size,
                                                   int voffset, int soffset, int offset,
                                                   int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// Raw (unformatted, stride 0) buffer resource over `bytes` bytes at `base`.
__device__ inline i32x4 make_buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = (int)bytes;
  r[3] = 0x00020000;  // raw 32-bit data format
  return r;
}

// Lane l's 16 bytes at rsrc + soffset + voffset land at LDS address lds + 16 l.
__device__ inline void dma16(const i32x4& rsrc, lds_void* lds, int voffset, int soffset) {
  bsa_raw_buffer_load_lds(rsrc, lds, 16, voffset, soffset, 0, 0);
}

// The same load written out by hand, for loops that wait for their tile loads
// themselves. The compiler does not see it as a memory request: it inserts no
// waits for it (a compiler-tracked LDS load makes every later LDS read wait
// for all loads in flight, since it cannot tell the target buffers apart), so
// the caller must wait (s_waitcnt vmcnt) and synchronise before reading the
// data. M0 holds the LDS destination; the s_nop covers the wait states the
// hardware requires after M0 and SGPR-operand writes.
__device__ inline void dma16_manual(const i32x4& rsrc, uint32_t lds_addr, int voffset,
                                    int soffset) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 4\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds_addr),
      "v"(voffset), "s"(rsrc), "s"(soffset)
      : "memory");
}
// 4 bytes per lane: lane l's dword lands at lds_addr + 4 l.
__device__ inline void dma4_manual(const i32x4& rsrc, uint32_t lds_addr, int voffset,
                                   int soffset) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 4\n\t"
      "buffer_load_dword %1, %2, %3 offen lds" ::"s"(lds_addr),
      "v"(voffset), "s"(rsrc), "s"(soffset)
      : "memory");
}
__device__ inline uint32_t lds_addr_of(const void* p) {
  return (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)reinterpret_cast<uintptr_t>(p));
}

}  // namespace bsa

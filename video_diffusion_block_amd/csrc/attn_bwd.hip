// Block-sparse attention backward.
//
// Prism trains with its block sparse attention (Prism page,
// trawling.dev/post/2299: sections on block composition and on the training
// procedure), so the selected-block attention needs gradients. With
// P_nm = exp(Q_n . K_m * scale - lse_n) over the forward's (query, key) pairs:
//   D_n = dO_n . O_n,  dV_m = sum_n P_nm dO_n,  dS_nm = P_nm (dO_n . V_m - D_n),
//   dQ_n = scale sum_m dS_nm K_m,  dK_m = scale sum_n dS_nm Q_n.
//
// Gradients are accumulated and returned in fp32 whatever the input dtype.
// dK/dV are accumulated key-major: the query-major lists are transposed into
// key-major lists (for each key block, the ascending query blocks that chose
// it), through a per-head bitmap, so every gradient row is owned by exactly
// one thread and summed in a fixed order (no atomics, bitwise reproducible).
#include "attn_common.hpp"
#include "kernels.hpp"

namespace bsa {
namespace {

// ------------------------------------------------------ D = rowsum(dO * O) --
template <typename T>
__global__ __launch_bounds__(256) void delta_kernel(const T* op, const T* dop, int d,
                                                    long long rows, float* delta) {
  const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  float acc = 0.f;
  for (int e = lane; e < d; e += 64) acc += to_f32(op[r * d + e]) * to_f32(dop[r * d + e]);
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) delta[r] = acc;
}

// ------------------------------------------------ list transpose (CSR->CSC) --
// bitmap[h][i][w] bit b: key block 32w+b is in the list of query block i.
__global__ __launch_bounds__(256) void bitmap_kernel(Lay L, const int32_t* counts,
                                                     const int32_t* idx, int words,
                                                     uint32_t* bitmap) {
  const int i = blockIdx.x, h = blockIdx.y;
  const size_t row = (size_t)h * L.M + i;
  uint32_t* out = bitmap + row * words;
  for (int w = threadIdx.x; w < words; w += 256) out[w] = 0u;
  __syncthreads();
  const int n = counts[row];
  const int32_t* lst = idx + row * L.M;
  for (int t = threadIdx.x; t < n; t += 256) {
    const int j = lst[t];
    atomicOr(out + (j >> 5), 1u << (j & 31));
  }
}

// For key block j: ascending query blocks whose lists hold j.
__global__ __launch_bounds__(256) void transpose_kernel(Lay L, const uint32_t* bitmap, int words,
                                                        int32_t* tcounts, int32_t* tidx) {
  __shared__ int wsum[4];
  __shared__ int base;
  const int j = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const size_t row = (size_t)h * L.M + j;
  int32_t* out = tidx + row * L.M;
  if (tid == 0) base = 0;
  __syncthreads();
  for (int i0 = 0; i0 < L.M; i0 += 256) {
    const int i = i0 + tid;
    const bool hit =
        i < L.M && ((bitmap[((size_t)h * L.M + i) * words + (j >> 5)] >> (j & 31)) & 1u);
    const unsigned long long ball = __ballot(hit);
    const int before_in_wave = __popcll(ball & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wv] = __popcll(ball);
    __syncthreads();
    int off = base;
    for (int v = 0; v < wv; ++v) off += wsum[v];
    if (hit) out[off + before_in_wave] = i;
    __syncthreads();
    if (tid == 0) base += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  if (tid == 0) tcounts[row] = base;
}

// ------------------------------------------------------------ dK/dV, scalar --
template <typename T, int D>
__global__ __launch_bounds__(128) void dkdv_scalar(Lay L, const int32_t* zone_shape, const T* qp,
                                                   const T* kp, const T* vp, const T* dop,
                                                   const float* lse, const float* delta,
                                                   const int32_t* tcounts, const int32_t* tidx,
                                                   float scale, float* dkp, float* dvp) {
  extern __shared__ float smem[];
  float* qs = smem;              // [B][D]
  float* ds = smem + L.B * D;    // [B][D] dO rows
  float* ls = ds + L.B * D;      // [B] lse
  float* dl = ls + L.B;          // [B] delta
  const int j = blockIdx.x, h = blockIdx.y, c = threadIdx.x;
  const size_t row = (size_t)h * L.M + j;
  const size_t koff = ((size_t)h * L.Np + (size_t)j * L.B + c) * D;
  const Box xj = block_box(L, zone_shape, j);
  const bool real = slot_real(xj, c);
  float k[D], v[D], dk[D], dv[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    k[e] = to_f32(kp[koff + e]);
    v[e] = to_f32(vp[koff + e]);
    dk[e] = 0.f;
    dv[e] = 0.f;
  }
  const int n = tcounts[row];
  const int32_t* lst = tidx + row * L.M;
  for (int it = 0; it < n; ++it) {
    const int i = lst[it];
    const Box xi = block_box(L, zone_shape, i);
    const size_t qoff = ((size_t)h * L.Np + (size_t)i * L.B) * D;
    __syncthreads();
    for (int e = c; e < L.B * D; e += blockDim.x) {
      qs[e] = to_f32(qp[qoff + e]);
      ds[e] = to_f32(dop[qoff + e]);
    }
    for (int e = c; e < L.B; e += blockDim.x) {
      ls[e] = lse[(size_t)h * L.Np + (size_t)i * L.B + e];
      dl[e] = delta[(size_t)h * L.Np + (size_t)i * L.B + e];
    }
    __syncthreads();
    if (!real) continue;
    for (int r = 0; r < L.B; ++r) {
      if (!slot_real(xi, r)) continue;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) {
        s = fmaf(qs[r * D + e], k[e], s);
        dp = fmaf(ds[r * D + e], v[e], dp);
      }
      const float p = expf(s * scale - ls[r]);
      const float dsc = p * (dp - dl[r]) * scale;
#pragma unroll
      for (int e = 0; e < D; ++e) {
        dv[e] = fmaf(p, ds[r * D + e], dv[e]);
        dk[e] = fmaf(dsc, qs[r * D + e], dk[e]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < D; ++e) {
    dkp[koff + e] = real ? dk[e] : 0.f;
    dvp[koff + e] = real ? dv[e] : 0.f;
  }
}

// --------------------------------------------------------------- dQ, scalar --
template <typename T, int D>
__global__ __launch_bounds__(128) void dq_scalar(Lay L, const int32_t* zone_shape, const T* qp,
                                                 const T* kp, const T* vp, const T* dop,
                                                 const float* lse, const float* delta,
                                                 const int32_t* counts, const int32_t* idx,
                                                 float scale, float* dqp) {
  extern __shared__ float smem[];
  float* ks = smem;              // [B][D]
  float* vs = smem + L.B * D;    // [B][D]
  const int i = blockIdx.x, h = blockIdx.y, r = threadIdx.x;
  const size_t row = (size_t)h * L.M + i;
  const size_t qoff = ((size_t)h * L.Np + (size_t)i * L.B + r) * D;
  const Box xi = block_box(L, zone_shape, i);
  const bool real = slot_real(xi, r);
  float q[D], dO[D], dq[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = to_f32(qp[qoff + e]);
    dO[e] = to_f32(dop[qoff + e]);
    dq[e] = 0.f;
  }
  const float lr = lse[(size_t)h * L.Np + (size_t)i * L.B + r];
  const float dr = delta[(size_t)h * L.Np + (size_t)i * L.B + r];
  const int n = counts[row];
  const int32_t* lst = idx + row * L.M;
  for (int it = 0; it < n; ++it) {
    const int j = lst[it];
    const Box xj = block_box(L, zone_shape, j);
    const size_t koff = ((size_t)h * L.Np + (size_t)j * L.B) * D;
    __syncthreads();
    for (int e = r; e < L.B * D; e += blockDim.x) {
      ks[e] = to_f32(kp[koff + e]);
      vs[e] = to_f32(vp[koff + e]);
    }
    __syncthreads();
    if (!real) continue;
    for (int c = 0; c < L.B; ++c) {
      if (!slot_real(xj, c)) continue;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) {
        s = fmaf(q[e], ks[c * D + e], s);
        dp = fmaf(dO[e], vs[c * D + e], dp);
      }
      const float p = expf(s * scale - lr);
      const float dsc = p * (dp - dr) * scale;
#pragma unroll
      for (int e = 0; e < D; ++e) dq[e] = fmaf(dsc, ks[c * D + e], dq[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < D; ++e) dqp[qoff + e] = real ? dq[e] : 0.f;
}

template <typename T, int D>
hipError_t launch_bwd_scalar(const Lay& L, const int32_t* zs, const T* q, const T* k, const T* v,
                             const T* dO, const float* lse, const float* delta,
                             const int32_t* counts, const int32_t* idx, const int32_t* tcounts,
                             const int32_t* tidx, int heads, float scale, float* dq, float* dk,
                             float* dv, hipStream_t st) {
  dim3 grid(L.M, heads);
  const size_t sh_kv = (2 * (size_t)L.B * D + 2 * (size_t)L.B) * sizeof(float);
  auto k1 = dkdv_scalar<T, D>;
  hipFuncSetAttribute(reinterpret_cast<const void*>(k1),
                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh_kv);
  k1<<<grid, L.B, sh_kv, st>>>(L, zs, q, k, v, dO, lse, delta, tcounts, tidx, scale, dk, dv);
  const size_t sh_q = 2 * (size_t)L.B * D * sizeof(float);
  auto k2 = dq_scalar<T, D>;
  hipFuncSetAttribute(reinterpret_cast<const void*>(k2),
                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh_q);
  k2<<<grid, L.B, sh_q, st>>>(L, zs, q, k, v, dO, lse, delta, counts, idx, scale, dq);
  return hipGetLastError();
}

}  // namespace

// Workspace: delta [H, Np] f32 | bitmap [H, M, words] u32 | tcounts [H, M] | tidx [H, M, M]
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t attn_bwd_workspace(const Lay& L, int heads, int d) {
  (void)d;
  const size_t words = (L.M + 31) / 32;
  return align256((size_t)heads * L.Np * sizeof(float)) +
         align256((size_t)heads * L.M * words * sizeof(uint32_t)) +
         align256((size_t)heads * L.M * sizeof(int32_t)) +
         align256((size_t)heads * L.M * L.M * sizeof(int32_t));
}

hipError_t launch_attn_bwd(const Lay& L, const int32_t* zone_shape, const void* qp,
                           const void* kp, const void* vp, const void* op, const void* dop,
                           const float* lse, const int32_t* counts, const int32_t* idx,
                           int heads, int d, bool bf16, float scale, void* dqp, void* dkp,
                           void* dvp, void* ws, hipStream_t st) {
  const int words = (L.M + 31) / 32;
  char* p = static_cast<char*>(ws);
  float* delta = reinterpret_cast<float*>(p);
  p += align256((size_t)heads * L.Np * sizeof(float));
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)heads * L.M * words * sizeof(uint32_t));
  int32_t* tcounts = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)heads * L.M * sizeof(int32_t));
  int32_t* tidx = reinterpret_cast<int32_t*>(p);

  const long long rows = (long long)heads * L.Np;
  const unsigned dgrid = (unsigned)((rows + 3) / 4);
  if (bf16)
    delta_kernel<__bf16><<<dgrid, 256, 0, st>>>(static_cast<const __bf16*>(op),
                                                  static_cast<const __bf16*>(dop), d, rows, delta);
  else
    delta_kernel<float><<<dgrid, 256, 0, st>>>(static_cast<const float*>(op),
                                                 static_cast<const float*>(dop), d, rows, delta);
  bitmap_kernel<<<dim3(L.M, heads), 256, 0, st>>>(L, counts, idx, words, bitmap);
  transpose_kernel<<<dim3(L.M, heads), 256, 0, st>>>(L, bitmap, words, tcounts, tidx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

#define BSA_BWD(T, D)                                                                        \
  return launch_bwd_scalar<T, D>(                                                            \
      L, zone_shape, static_cast<const T*>(qp), static_cast<const T*>(kp),                   \
      static_cast<const T*>(vp), static_cast<const T*>(dop), lse, delta, counts, idx, tcounts, \
      tidx, heads, scale, static_cast<float*>(dqp), static_cast<float*>(dkp),                  \
      static_cast<float*>(dvp), st)
  if (bf16) {
    if (d == 64) BSA_BWD(__bf16, 64);
    BSA_BWD(__bf16, 128);
  }
  if (d == 64) BSA_BWD(float, 64);
  BSA_BWD(float, 128);
#undef BSA_BWD
}

}  // namespace bsa

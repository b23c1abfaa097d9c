// Block-mean pooling and hybrid block selection.
//
// Prism page (trawling.dev/post/2299), section on block composition matched to
// regional information: block-level features drive a hybrid block selection
// that sets each query's sparsity dynamically (configuration examples: sparsity
// 0.75/0.80/0.85/0.93, CDF threshold 0.20). Reading implemented: block means of
// the real tokens; pooled logits qbar_i . kbar_j / sqrt(d) over non-empty key
// blocks; order by logit descending (lower id first on equal logits); keep the
// first max(k, m) blocks, k = max(1, ceil(M_v (1 - s))) and m the shortest
// prefix whose softmax mass reaches tau; emit them in ascending id.
//
// All of it runs in fp64: pooled logits of neighbouring blocks can differ by
// less than fp32 resolution, and the list must match an fp64 evaluation of the
// rule except at near-ties. Cost is small next to attention (C5-size: 4 heads
// x 1920^2 x 128 fp64 FMAs).
#include <float.h>
#include <math.h>

#include "attn_common.hpp"
#include "kernels.hpp"

namespace bsa {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- pooling --
template <typename T, int EPC>  // EPC: elements per 16-byte chunk
__global__ __launch_bounds__(kThreads) void pool_kernel(Lay L, const BlockMeta* __restrict__ meta,
                                                        const T* __restrict__ qp,
                                                        const T* __restrict__ kp, int d,
                                                        double* __restrict__ qbar,
                                                        double* __restrict__ kbar) {
  extern __shared__ double red[];  // [groups][d]
  const int b = blockIdx.x, h = blockIdx.y;
  const T* __restrict__ src = blockIdx.z ? kp : qp;
  double* __restrict__ out = blockIdx.z ? kbar : qbar;
  const BlockMeta& mb = meta[b];
  const int cnt = mb.count();
  const int chunks = d / EPC;
  const int groups = kThreads / chunks;
  const int c = threadIdx.x % chunks, g = threadIdx.x / chunks;
  double acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.0;
  const T* base = src + ((size_t)h * L.Np + (size_t)b * L.B) * d + c * EPC;
  // all of this thread's rows are loaded before any is summed (latency overlap);
  // pad slots are skipped by the block's real-slot mask
  constexpr int kMaxRows = 16;
  u32x4 raw[kMaxRows];
  const int nrows = L.B / groups;
#pragma unroll
  for (int k = 0; k < kMaxRows; ++k)
    if (k < nrows) raw[k] = *reinterpret_cast<const u32x4*>(base + (size_t)(g + k * groups) * d);
#pragma unroll
  for (int k = 0; k < kMaxRows; ++k) {
    const int r = g + k * groups;
    if (k < nrows && ((mb.mask(r >> 5) >> (r & 31)) & 1u)) {
      const T* v = reinterpret_cast<const T*>(&raw[k]);
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[e] += (double)(float)v[e];
    }
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) red[g * d + c * EPC + e] = acc[e];
  __syncthreads();
  for (int e = threadIdx.x; e < d; e += kThreads) {
    double s = 0.0;
    for (int gg = 0; gg < groups; ++gg) s += red[gg * d + e];
    out[((size_t)h * L.M + b) * d + e] = cnt ? s / (double)cnt : 0.0;
  }
}

// --------------------------------------------------------- pooled logits --
constexpr int kLT = 64;  // output tile
constexpr int kLE = 16;  // reduction chunk

__global__ __launch_bounds__(kThreads) void pooled_logits_kernel(Lay L,
                                                                 const BlockMeta* __restrict__ meta,
                                                                 const double* __restrict__ qbar,
                                                                 const double* __restrict__ kbar,
                                                                 int d, double scale,
                                                                 double* __restrict__ logits) {
  __shared__ double qs[kLE][kLT + 1];
  __shared__ double ks[kLE][kLT + 1];
  const int i0 = blockIdx.x * kLT, j0 = blockIdx.y * kLT, h = blockIdx.z;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const double* qh = qbar + (size_t)h * L.M * d;
  const double* kh = kbar + (size_t)h * L.M * d;
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  for (int e0 = 0; e0 < d; e0 += kLE) {
    for (int t = threadIdx.x; t < kLT * kLE; t += kThreads) {
      const int r = t / kLE, e = t % kLE;
      qs[e][r] = (i0 + r < L.M) ? qh[(size_t)(i0 + r) * d + e0 + e] : 0.0;
      ks[e][r] = (j0 + r < L.M) ? kh[(size_t)(j0 + r) * d + e0 + e] : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kLE; ++e) {
      double av[4], bv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) av[a] = qs[e][ty + 16 * a];
#pragma unroll
      for (int b = 0; b < 4; ++b) bv[b] = ks[e][tx + 16 * b];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fma(av[a], bv[b], acc[a][b]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int j = j0 + tx + 16 * b;
    if (j >= L.M) continue;
    const bool key_ok = meta[j].count() > 0;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int i = i0 + ty + 16 * a;
      if (i >= L.M) continue;
      logits[((size_t)h * L.M + i) * L.M + j] = key_ok ? acc[a][b] * scale : -INFINITY;
    }
  }
}

// -------------------------------------------------------------- selection --
__device__ inline bool before(double ka, int ia, double kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// Block-wide sums over kThreads threads (fp64 / int).
__device__ inline double block_sum(double v, double* sh) {
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
    __syncthreads();
  }
  const double r = sh[0];
  __syncthreads();
  return r;
}

template <int P2>
__global__ __launch_bounds__(kThreads) void select_kernel(Lay L, const BlockMeta* __restrict__ meta,
                                                          const double* __restrict__ logits,
                                                          int sparsity_1e4, double tau,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ idx) {
  constexpr int E = P2 / kThreads;  // entries per thread in the scans
  __shared__ double key[P2];        // logits, then (after the sort) exp(l - max)
  __shared__ int id[P2];
  __shared__ int flag[P2];
  __shared__ double part[kThreads];
  __shared__ int ipart[kThreads];
  __shared__ int m_first;

  const int i = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const size_t row = (size_t)h * L.M + i;
  if (meta[i].count() == 0) {  // empty query block: empty list
    if (tid == 0) counts[row] = 0;
    return;
  }
  const double* lg = logits + row * L.M;
  int valid = 0;
  for (int j = tid; j < P2; j += kThreads) {
    double v = -INFINITY;
    if (j < L.M && meta[j].count() > 0) {
      v = lg[j];
      ++valid;
    }
    key[j] = v;
    id[j] = j;
    flag[j] = 0;
  }
  ipart[tid] = valid;
  if (tid == 0) m_first = INT_MAX;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (tid < s) ipart[tid] += ipart[tid + s];
    __syncthreads();
  }
  const int mv = ipart[0];

  // bitonic sort: logit descending, then block id ascending
  for (int k = 2; k <= P2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int t = tid; t < P2; t += kThreads) {
        const int u = t ^ j;
        if (u > t) {
          const double ka = key[t], kb = key[u];
          const int ia = id[t], ib = id[u];
          const bool up = (t & k) == 0;
          if (up ? before(kb, ib, ka, ia) : before(ka, ia, kb, ib)) {
            key[t] = kb; key[u] = ka;
            id[t] = ib; id[u] = ia;
          }
        }
      }
      __syncthreads();
    }
  }

  // softmax mass in sorted order, prefix-summed; m = first prefix reaching tau
  const double mx = key[0];
  __syncthreads();
  double z_loc = 0.0;
  for (int e = 0; e < E; ++e) {
    const int r = tid * E + e;
    const double ex = r < mv ? exp(key[r] - mx) : 0.0;
    key[r] = ex;
    z_loc += ex;
  }
  const double Z = block_sum(z_loc, part);
  double run = 0.0;
  for (int e = 0; e < E; ++e) run += key[tid * E + e] / Z;
  part[tid] = run;
  __syncthreads();
  if (tid == 0) {
    double acc = 0.0;
    for (int t = 0; t < kThreads; ++t) {
      const double v = part[t];
      part[t] = acc;
      acc += v;
    }
  }
  __syncthreads();
  double c = part[tid];
  for (int e = 0; e < E; ++e) {
    const int r = tid * E + e;
    if (r < mv) {
      c += key[r] / Z;
      if (c >= tau) {
        atomicMin(&m_first, r + 1);
        break;
      }
    }
  }
  __syncthreads();
  const int m = m_first == INT_MAX ? mv : m_first;
  const int k = max(1, (mv * (10000 - sparsity_1e4) + 9999) / 10000);
  const int n = min(max(k, m), mv);
  for (int r = tid; r < n; r += kThreads) flag[id[r]] = 1;
  __syncthreads();

  // ascending compaction of the flagged block ids
  int cnt = 0;
  for (int e = 0; e < E; ++e) cnt += flag[tid * E + e];
  ipart[tid] = cnt;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int t = 0; t < kThreads; ++t) {
      const int v = ipart[t];
      ipart[t] = acc;
      acc += v;
    }
  }
  __syncthreads();
  int pos = ipart[tid];
  int32_t* out = idx + row * L.M;
  for (int e = 0; e < E; ++e) {
    const int j = tid * E + e;
    if (flag[j]) out[pos++] = j;
  }
  if (tid == 0) counts[row] = n;
}

}  // namespace

hipError_t launch_pool(const Lay& L, const BlockMeta* meta, const void* qp, const void* kp,
                       int heads, int d, bool bf16, double* qbar, double* kbar, hipStream_t st) {
  dim3 grid(L.M, heads, 2);
  if (bf16) {
    const int groups = kThreads / (d / 8);
    pool_kernel<__bf16, 8><<<grid, kThreads, groups * d * sizeof(double), st>>>(
        L, meta, static_cast<const __bf16*>(qp), static_cast<const __bf16*>(kp), d, qbar, kbar);
  } else {
    const int groups = kThreads / (d / 4);
    pool_kernel<float, 4><<<grid, kThreads, groups * d * sizeof(double), st>>>(
        L, meta, static_cast<const float*>(qp), static_cast<const float*>(kp), d, qbar, kbar);
  }
  return hipGetLastError();
}

hipError_t launch_pooled_logits(const Lay& L, const BlockMeta* meta, const double* qbar,
                                const double* kbar, int heads, int d, double scale,
                                double* logits, hipStream_t st) {
  dim3 grid((L.M + kLT - 1) / kLT, (L.M + kLT - 1) / kLT, heads);
  pooled_logits_kernel<<<grid, kThreads, 0, st>>>(L, meta, qbar, kbar, d, scale, logits);
  return hipGetLastError();
}

hipError_t launch_select(const Lay& L, const BlockMeta* meta, const double* logits,
                         int heads, int sparsity_1e4, double tau, int32_t* counts, int32_t* idx,
                         hipStream_t st) {
  dim3 grid(L.M, heads);
#define BSA_SELECT(P)                                                                      \
  select_kernel<P><<<grid, kThreads, 0, st>>>(L, meta, logits, sparsity_1e4, tau,       \
                                              counts, idx)
  if (L.M <= 256) BSA_SELECT(256);
  else if (L.M <= 512) BSA_SELECT(512);
  else if (L.M <= 1024) BSA_SELECT(1024);
  else if (L.M <= 2048) BSA_SELECT(2048);
  else BSA_SELECT(4096);
#undef BSA_SELECT
  return hipGetLastError();
}

}  // namespace bsa

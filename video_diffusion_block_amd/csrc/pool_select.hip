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

// Wave-level sum / exclusive prefix sum / min over the 64 lanes, in a fixed
// order (the result does not depend on timing).
__device__ inline double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ inline int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ inline int wave_min(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
template <typename T>
__device__ inline T wave_exclusive_scan(T v, int lane) {
  T incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  return incl - v;
}

// Bitonic compare-exchange steps on a row held in registers: lane l holds
// sorted positions C l .. C l + C - 1 (element e at position C l + e). Within
// a lane the partner of e is e ^ JJ (JJ < C, known at compile time); across
// lanes the partner of lane l is lane l ^ (jj / C), same e. Positions whose
// bit k is clear are sorted into "before" order, the others reversed.
template <int C, int JJ>
__device__ inline void bitonic_in_lane(double (&key)[C], int (&id)[C], int lane, int k) {
#pragma unroll
  for (int e = 0; e < C; ++e) {
    if (e & JJ) continue;
    const int f = e | JJ;
    const bool up = ((lane * C + e) & k) == 0;
    const bool swap = up ? before(key[f], id[f], key[e], id[e])
                         : before(key[e], id[e], key[f], id[f]);
    const double ke = key[e], kf = key[f];
    const int ie = id[e], jf = id[f];
    key[e] = swap ? kf : ke;
    key[f] = swap ? ke : kf;
    id[e] = swap ? jf : ie;
    id[f] = swap ? ie : jf;
  }
}
template <int C>
__device__ inline void bitonic_cross_lane(double (&key)[C], int (&id)[C], int lane, int k, int jj) {
  const int lm = jj / C;
  const bool lower = (lane & lm) == 0;
  const bool up = ((lane * C) & k) == 0;  // bit k of the position (k > jj >= C)
  const bool keep_first = lower == up;
#pragma unroll
  for (int e = 0; e < C; ++e) {
    const double ko = __shfl_xor(key[e], lm);
    const int io = __shfl_xor(id[e], lm);
    const bool mine_first = before(key[e], id[e], ko, io);
    if (mine_first != keep_first) {
      key[e] = ko;
      id[e] = io;
    }
  }
}

// One wavefront per (head, query block) row, WAVES rows per workgroup. The
// row's P2 = 64 C entries (logit, block id) are sorted in registers by a
// bitonic network (lane-local steps and cross-lane exchanges), then scanned.
template <int P2, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void select_kernel(Lay L, const BlockMeta* __restrict__ meta,
                                                             const double* __restrict__ logits,
                                                             int sparsity_1e4, double tau,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ idx) {
  constexpr int C = P2 / 64;  // entries per lane
  __shared__ uint32_t sbits[WAVES][P2 / 32];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = blockIdx.x * WAVES + w, h = blockIdx.y;
  if (i >= L.M) return;  // (whole wavefront)
  const size_t row = (size_t)h * L.M + i;
  if (meta[i].count() == 0) {  // empty query block: empty list
    if (lane == 0) counts[row] = 0;
    return;
  }
  uint32_t* bits = sbits[w];
  const double* lg = logits + row * L.M;

  // candidates are the non-empty key blocks, whose pooled logits are finite
  double key[C];
  int id[C];
  int valid = 0;
#pragma unroll
  for (int e = 0; e < C; ++e) {
    const int j = lane * C + e;
    key[e] = j < L.M ? lg[j] : -INFINITY;
    id[e] = j;
    valid += key[e] != -INFINITY;
  }
#pragma unroll
  for (int e = lane; e < P2 / 32; e += 64) bits[e] = 0u;
  const int mv = wave_sum(valid);

  // bitonic sort: logit descending, then block id ascending
  for (int k = 2; k <= P2; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      if (jj >= C) {
        bitonic_cross_lane<C>(key, id, lane, k, jj);
      } else {
        switch (jj) {
          case 1: bitonic_in_lane<C, 1>(key, id, lane, k); break;
          case 2: bitonic_in_lane<C, (C > 2 ? 2 : 1)>(key, id, lane, k); break;
          case 4: bitonic_in_lane<C, (C > 4 ? 4 : 1)>(key, id, lane, k); break;
          case 8: bitonic_in_lane<C, (C > 8 ? 8 : 1)>(key, id, lane, k); break;
          case 16: bitonic_in_lane<C, (C > 16 ? 16 : 1)>(key, id, lane, k); break;
          default: bitonic_in_lane<C, (C > 32 ? 32 : 1)>(key, id, lane, k); break;
        }
      }
    }
  }

  // softmax mass in sorted order, prefix-summed; m = first prefix reaching tau
  const double mx = __shfl(key[0], 0);
  double* ex = key;  // exp(l - max) replaces the logits
  double z_loc = 0.0;
#pragma unroll
  for (int e = 0; e < C; ++e) {
    ex[e] = lane * C + e < mv ? exp(key[e] - mx) : 0.0;
    z_loc += ex[e];
  }
  const double Z = wave_sum(z_loc);
  double run = 0.0;
#pragma unroll
  for (int e = 0; e < C; ++e) run += ex[e] / Z;
  double c = wave_exclusive_scan(run, lane);
  int m_loc = INT_MAX;
#pragma unroll
  for (int e = 0; e < C; ++e) {
    const int r = lane * C + e;
    if (r < mv && m_loc == INT_MAX) {
      c += ex[e] / Z;
      if (c >= tau) m_loc = r + 1;
    }
  }
  const int m_first = wave_min(m_loc);
  const int m = m_first == INT_MAX ? mv : m_first;
  const int k = max(1, (mv * (10000 - sparsity_1e4) + 9999) / 10000);
  const int n = min(max(k, m), mv);
#pragma unroll
  for (int e = 0; e < C; ++e)
    if (lane * C + e < n) atomicOr(&bits[id[e] >> 5], 1u << (id[e] & 31));

  // ascending compaction of the selected block ids (lane l: ids C l .. C l + C - 1)
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < C; ++e) {
    const int b = lane * C + e;
    cnt += (bits[b >> 5] >> (b & 31)) & 1u;
  }
  int pos = wave_exclusive_scan(cnt, lane);
  int32_t* out = idx + row * L.M;
#pragma unroll
  for (int e = 0; e < C; ++e) {
    const int b = lane * C + e;
    if ((bits[b >> 5] >> (b & 31)) & 1u) out[pos++] = b;
  }
  if (lane == 0) counts[row] = n;
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
#define BSA_SELECT(P, W)                                                                   \
  select_kernel<P, W><<<dim3((L.M + (W) - 1) / (W), heads), 64 * (W), 0, st>>>(            \
      L, meta, logits, sparsity_1e4, tau, counts, idx)
  if (L.M <= 256) BSA_SELECT(256, 4);
  else if (L.M <= 512) BSA_SELECT(512, 4);
  else if (L.M <= 1024) BSA_SELECT(1024, 4);
  else if (L.M <= 2048) BSA_SELECT(2048, 4);
  else BSA_SELECT(4096, 2);
#undef BSA_SELECT
  return hipGetLastError();
}

}  // namespace bsa

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
// rule except at near-ties. Cost is small next to attention (2K workload: 4 heads
// x 1920^2 x 128 fp64 FMAs, on the fp64 matrix cores).
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
// l[h,i,j] = qbar_i . kbar_j * scale on fp64 MFMA (v_mfma_f64_16x16x4_f64).
// One workgroup of 4 wavefronts per 64 x 64 tile of (query block, key block);
// wavefront w owns the 32 x 32 sub-tile (w / 2, w % 2) as 2 x 2 MFMA tiles.
// The reduction over d runs in chunks of 16 staged in LDS ([k][row] layout,
// padded rows) and in k-steps of 4 inside a chunk.
// Operand layout of the 16x16x4 fp64 product: lane l supplies A[l % 16][l / 16]
// and B[l / 16][l % 16]; accumulator element r of lane l is D[4 r + l / 16][l % 16]
// (probed on gfx950).
constexpr int kPT = 64;  // output tile
constexpr int kPE = 16;  // reduction chunk
typedef double f64x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void pooled_logits_kernel(Lay L,
                                                                 const BlockMeta* __restrict__ meta,
                                                                 const double* __restrict__ qbar,
                                                                 const double* __restrict__ kbar,
                                                                 int d, double scale,
                                                                 double* __restrict__ logits) {
  __shared__ double sq[kPE][kPT + 1];
  __shared__ double sk[kPE][kPT + 1];
  const int i0 = blockIdx.x * kPT, j0 = blockIdx.y * kPT, h = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wi = 32 * (w >> 1), wj = 32 * (w & 1);
  const int l16 = lane & 15, kq = lane >> 4;
  const double* qh = qbar + (size_t)h * L.M * d;
  const double* kh = kbar + (size_t)h * L.M * d;
  f64x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
  const int le = threadIdx.x & (kPE - 1), lr = threadIdx.x / kPE;  // loader: element, row
  constexpr int kLd = kPT * kPE / kThreads;                         // loads per operand and lane
  // the next chunk's operands are loaded into registers while this one is
  // multiplied
  double nq[kLd], nk[kLd];
  auto gload = [&](int e0) {
#pragma unroll
    for (int u = 0; u < kLd; ++u) {
      const int r = lr + (kThreads / kPE) * u;
      nq[u] = (i0 + r < L.M) ? qh[(size_t)(i0 + r) * d + e0 + le] : 0.0;
      nk[u] = (j0 + r < L.M) ? kh[(size_t)(j0 + r) * d + e0 + le] : 0.0;
    }
  };
  gload(0);
  for (int e0 = 0; e0 < d; e0 += kPE) {
#pragma unroll
    for (int u = 0; u < kLd; ++u) {
      const int r = lr + (kThreads / kPE) * u;
      sq[le][r] = nq[u];
      sk[le][r] = nk[u];
    }
    __syncthreads();
    if (e0 + kPE < d) gload(e0 + kPE);
#pragma unroll
    for (int ks = 0; ks < kPE / 4; ++ks) {
      const int kk = 4 * ks + kq;
      double av[2], bv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        av[t] = sq[kk][wi + 16 * t + l16];
        bv[t] = sk[kk][wj + 16 * t + l16];
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int j = j0 + wj + 16 * b + l16;
    if (j >= L.M) continue;
    const bool key_ok = meta[j].count() > 0;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + wi + 16 * a + 4 * r + kq;
        if (i < L.M) logits[((size_t)h * L.M + i) * L.M + j] = key_ok ? acc[a][b][r] * scale : -INFINITY;
      }
  }
}

// -------------------------------------------------------------- selection --
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
__device__ inline double wave_max(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}
// Order-preserving map of a finite double to uint64, reversed: a smaller key
// is a larger logit.
__device__ inline uint64_t rank_key(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint64_t mono = (b >> 63) ? ~b : (b | 0x8000000000000000ull);
  return ~mono;
}
// The full key of the one candidate whose top bits (those at and above
// `shift`) equal `prefix` (a bin that holds exactly one element).
template <int C>
__device__ inline uint64_t sole_key(const double (&key)[C], uint64_t prefix, int shift) {
  const uint64_t mask = ~0ull << shift;
  uint64_t mine = 0;
  bool have = false;
#pragma unroll
  for (int e = 0; e < C; ++e) {
    if (key[e] != -INFINITY) {
      const uint64_t u = rank_key(key[e]);
      if ((u & mask) == prefix) {
        mine = u;
        have = true;
      }
    }
  }
  const int src = __ffsll((long long)__ballot(have)) - 1;
  const uint32_t lo = __shfl((uint32_t)mine, src), hi = __shfl((uint32_t)(mine >> 32), src);
  return ((uint64_t)hi << 32) | lo;
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

// One wavefront per (head, query block) row, WAVES rows per workgroup; lane l
// holds the row's logits of key blocks P2/64 l .. P2/64 (l + 1) - 1 in
// registers (P2: a multiple of 64 at least the block count). No sort: the cut of the order (logit descending, id ascending) is
// found by MSB-first radix selection on an order-preserving 64-bit key (eight
// 8-bit digits, LDS histograms, wave scans), first for rank k; when the top-k
// set already holds probability mass >= tau it is the list, otherwise a second
// selection finds the element at which the mass in that order reaches tau (bins
// carry the mass as well), and the list is everything up to it. Equal logits at
// a cut are taken in id order. The selected ids are compacted in ascending
// order through an LDS bitmap and a wave scan.
template <int P2, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void select_kernel(Lay L, const BlockMeta* __restrict__ meta,
                                                             const double* __restrict__ logits,
                                                             int sparsity_1e4, double tau,
                                                             int frames_per_chunk,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ idx) {
  constexpr int C = P2 / 64;  // entries per lane
  __shared__ uint32_t sbits[WAVES][P2 / 32];
  __shared__ uint32_t shist[WAVES][256];
  __shared__ double smass[WAVES][256];
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

  // candidates are the non-empty key blocks, whose pooled logits are finite.
  // Frame-chunk causal rows (frames_per_chunk > 0, a multiple of the zone's
  // time extent): chunk(b) = first frame of b's zone / F, and since zones run
  // time-slowest the blocks of chunks <= chunk(i) are the prefix of ids below
  // the first zone of chunk(i) + 1.
  int jend = L.M;
  if (frames_per_chunk > 0) {
    const int zrow = (i / L.bpz) / (L.gzh * L.gzw);  // zone row (in time) of i
    const long long next_row =
        (long long)((zrow * L.zt) / frames_per_chunk + 1) * frames_per_chunk / L.zt;
    const long long end = next_row * L.gzh * L.gzw * L.bpz;
    jend = end < L.M ? (int)end : L.M;
  }
  double key[C];
  int id[C];
  int valid = 0;
#pragma unroll
  for (int e = 0; e < C; ++e) {
    const int j = lane * C + e;
    key[e] = j < jend ? lg[j] : -INFINITY;
    id[e] = j;
    valid += key[e] != -INFINITY;
  }
#pragma unroll
  for (int e = lane; e < P2 / 32; e += 64) bits[e] = 0u;
  const int mv = wave_sum(valid);
  const int k_top = max(1, (mv * (10000 - sparsity_1e4) + 9999) / 10000);

  // The top-k set from a radix select of the k-th best (logit descending,
  // then id ascending); when its softmax mass reaches tau the CDF prefix is
  // inside it and the list is the top-k set.
  {
    uint32_t* hist = shist[w];
    double mloc = -INFINITY;
#pragma unroll
    for (int e = 0; e < C; ++e) mloc = fmax(mloc, key[e]);
    const double mx = wave_max(mloc);
    uint64_t prefix = 0;
    int remaining = k_top;  // rank still to find inside the current prefix
    int count_eq = 0;       // elements equal to the final prefix
#pragma unroll 1
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      const uint64_t above = pass ? ~0ull << (shift + 8) : 0ull;
#pragma unroll
      for (int b = lane; b < 256; b += 64) hist[b] = 0u;
#pragma unroll
      for (int e = 0; e < C; ++e) {
        if (key[e] != -INFINITY) {
          const uint64_t u = rank_key(key[e]);
          if ((u & above) == prefix) atomicAdd(&hist[(u >> shift) & 255], 1u);
        }
      }
      const uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2],
                     c3 = hist[4 * lane + 3];
      const int local = (int)(c0 + c1 + c2 + c3);
      const int before = wave_exclusive_scan(local, lane);
      // the lane whose four bins hold the rank
      const bool here = before < remaining && remaining <= before + local;
      const uint64_t ball = __ballot(here);
      const int src = __ffsll((long long)ball) - 1;
      // within the lane: the first bin whose cumulative count reaches the rank
      int digit = 0, cb = 0, ce = 0;
      {
        const int cs[4] = {(int)c0, (int)c1, (int)c2, (int)c3};
        int acc = before;
        bool got = false;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (!got && remaining <= acc + cs[q]) {
            got = true;
            digit = 4 * lane + q;
            cb = acc;
            ce = cs[q];
          }
          acc += cs[q];
        }
      }
      digit = __shfl(digit, src);
      cb = __shfl(cb, src);
      ce = __shfl(ce, src);
      prefix |= (uint64_t)digit << shift;
      remaining -= cb;
      count_eq = ce;
      if (ce == 1) {  // one element left in range: it is the cut (later
        prefix = sole_key(key, prefix, shift);  // passes would only confirm it)
        break;
      }
    }
    // ties on the logit: the `remaining` smallest ids among the equal ones
    int id_cut = INT_MAX;
    if (remaining < count_eq) {
      int cur = -1;
#pragma unroll 1
      for (int r = 0; r < remaining; ++r) {
        int mn = INT_MAX;
#pragma unroll
        for (int e = 0; e < C; ++e)
          if (key[e] != -INFINITY && rank_key(key[e]) == prefix && id[e] > cur) mn = min(mn, id[e]);
        cur = wave_min(mn);
      }
      id_cut = cur;
    }
    double zl = 0.0, ml = 0.0;
#pragma unroll
    for (int e = 0; e < C; ++e) {
      if (key[e] != -INFINITY) {
        const double ex = exp(key[e] - mx);
        const uint64_t u = rank_key(key[e]);
        zl += ex;
        if (u < prefix || (u == prefix && id[e] <= id_cut)) ml += ex;
      }
    }
    const double Z = wave_sum(zl);
    const double mass = wave_sum(ml) / Z;
    // the top-k cut, kept in case the CDF crossing falls inside the top-k set
    const uint64_t prefix_k = prefix;
    const int id_cut_k = id_cut;
    if (mass < tau) {
      // The CDF prefix is longer than k: a second radix select, now of the
      // first element at which the mass in (logit desc, id asc) order reaches
      // tau; bins carry counts and probability mass.
      double* hm = smass[w];
      prefix = 0;
      double mbefore = 0.0;  // mass of the elements ranked before the prefix range
      int cbefore = 0;       // their count
      count_eq = 0;
#pragma unroll 1
      for (int pass = 0; pass < 8; ++pass) {
        const int shift = 56 - 8 * pass;
        const uint64_t above = pass ? ~0ull << (shift + 8) : 0ull;
#pragma unroll
        for (int b = lane; b < 256; b += 64) {
          hist[b] = 0u;
          hm[b] = 0.0;
        }
#pragma unroll
        for (int e = 0; e < C; ++e) {
          if (key[e] != -INFINITY) {
            const uint64_t u = rank_key(key[e]);
            if ((u & above) == prefix) {
              atomicAdd(&hist[(u >> shift) & 255], 1u);
              atomicAdd(&hm[(u >> shift) & 255], exp(key[e] - mx) / Z);
            }
          }
        }
        const int cs[4] = {(int)hist[4 * lane], (int)hist[4 * lane + 1], (int)hist[4 * lane + 2],
                           (int)hist[4 * lane + 3]};
        const double ms[4] = {hm[4 * lane], hm[4 * lane + 1], hm[4 * lane + 2], hm[4 * lane + 3]};
        const double lm = (ms[0] + ms[1]) + (ms[2] + ms[3]);
        const int lc = cs[0] + cs[1] + cs[2] + cs[3];
        const double bm = mbefore + wave_exclusive_scan(lm, lane);
        const int bc = cbefore + wave_exclusive_scan(lc, lane);
        // the bin holding the crossing: the first whose cumulative mass reaches
        // tau; if rounding left this range's total just under tau (the bins'
        // sums regroup the previous pass's), its last non-empty bin
        const bool here = bm < tau && tau <= bm + lm;
        const uint64_t ball = __ballot(here);
        const uint64_t nonempty = __ballot(lc > 0);
        const int src = ball ? __ffsll((long long)ball) - 1 : 63 - __clzll((long long)nonempty);
        int digit = 0, cbin = bc, ceq = 0;
        double mbin = bm;
        {
          double acc = bm;
          int accc = bc;
          bool got = false;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const bool take = ball ? (!got && cs[q] > 0 && tau <= acc + ms[q]) : cs[q] > 0;
            if (take) {
              got = true;
              digit = 4 * lane + q;
              mbin = acc;
              cbin = accc;
              ceq = cs[q];
            }
            acc += ms[q];
            accc += cs[q];
          }
        }
        digit = __shfl(digit, src);
        mbefore = __shfl(mbin, src);
        cbefore = __shfl(cbin, src);
        count_eq = __shfl(ceq, src);
        prefix |= (uint64_t)digit << shift;
        if (count_eq == 1) {  // as above: the crossing is this one element
          prefix = sole_key(key, prefix, shift);
          break;
        }
      }
      // equal logits at the crossing: take them in id order until tau
      int cut = INT_MAX, taken = count_eq;
      if (count_eq > 1) {
        int cur = -1;
        double acc = mbefore;
        taken = 0;
#pragma unroll 1
        for (int r = 0; r < count_eq; ++r) {
          int mn = INT_MAX;
          double pe = 0.0;
#pragma unroll
          for (int e = 0; e < C; ++e)
            if (key[e] != -INFINITY && rank_key(key[e]) == prefix && id[e] > cur && id[e] < mn) {
              mn = id[e];
              pe = exp(key[e] - mx) / Z;
            }
          const int mw = wave_min(mn);
          const uint64_t own = __ballot(mn == mw && mn != INT_MAX);
          pe = __shfl(pe, __ffsll((long long)own) - 1);
          cur = mw;
          acc += pe;
          ++taken;
          if (acc >= tau) break;
        }
        cut = cur;
      }
      const int m_cdf = cbefore + taken;
      if (m_cdf > k_top) {
        id_cut = cut;  // the list: every element ranked up to the crossing
      } else {
        // Both sets are prefixes of one order, so the union is the longer
        // one. Pass 1 found the top-k mass below tau, so the crossing should
        // lie past rank k; the mass sums of the two passes group the same
        // terms differently, and when the top-k mass is within rounding of tau
        // the second pass can place the crossing inside the top-k set. The
        // list is then the top-k set.
        prefix = prefix_k;
        id_cut = id_cut_k;
      }
    }
    {
#pragma unroll
      for (int e = 0; e < C; ++e) {
        if (key[e] != -INFINITY) {
          const uint64_t u = rank_key(key[e]);
          if (u < prefix || (u == prefix && id[e] <= id_cut))
            atomicOr(&bits[id[e] >> 5], 1u << (id[e] & 31));
        }
      }
      int cnt = 0;
#pragma unroll
      for (int e = 0; e < C; ++e) {
        const int b = lane * C + e;
        cnt += (bits[b >> 5] >> (b & 31)) & 1u;
      }
      int pos = wave_exclusive_scan(cnt, lane);
      // the count is the number of ids written (the length of the prefix
      // the cut marks), so the list and its count cannot disagree
      const int n_sel = wave_sum(cnt);
      int32_t* out = idx + row * L.M;
#pragma unroll
      for (int e = 0; e < C; ++e) {
        const int b = lane * C + e;
        if ((bits[b >> 5] >> (b & 31)) & 1u) out[pos++] = b;
      }
      if (lane == 0) counts[row] = n_sel;
    }
  }

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
  dim3 grid((L.M + kPT - 1) / kPT, (L.M + kPT - 1) / kPT, heads);
  pooled_logits_kernel<<<grid, kThreads, 0, st>>>(L, meta, qbar, kbar, d, scale, logits);
  return hipGetLastError();
}

hipError_t launch_select(const Lay& L, const BlockMeta* meta, const double* logits,
                         int heads, int sparsity_1e4, double tau, int32_t* counts, int32_t* idx,
                         hipStream_t st, int frames_per_chunk) {
#define BSA_SELECT(P, W)                                                                   \
  select_kernel<P, W><<<dim3((L.M + (W) - 1) / (W), heads), 64 * (W), 0, st>>>(            \
      L, meta, logits, sparsity_1e4, tau, frames_per_chunk, counts, idx)
  // row widths: multiples of 64 (one register slot per lane each), chosen
  // to cover the common block counts with few empty slots
  if (L.M <= 256) BSA_SELECT(256, 4);
  else if (L.M <= 512) BSA_SELECT(512, 4);
  else if (L.M <= 1024) BSA_SELECT(1024, 4);
  else if (L.M <= 1280) BSA_SELECT(1280, 4);
  else if (L.M <= 1536) BSA_SELECT(1536, 4);
  else if (L.M <= 1920) BSA_SELECT(1920, 4);
  else if (L.M <= 2048) BSA_SELECT(2048, 4);
  else if (L.M <= 3072) BSA_SELECT(3072, 2);
  else BSA_SELECT(4096, 2);
#undef BSA_SELECT
  return hipGetLastError();
}

}  // namespace bsa

// Token <-> block-order gather/scatter.
//
// Prism page (trawling.dev/post/2299), section on block composition matched to
// regional information: tokens of a macro-zone are regrouped into blocks of the
// zone's shape. One workgroup moves one (block, head, tensor) tile: B rows of
// d elements, 16 bytes per lane per step. Source rows of a block come in runs
// of bw consecutive raster tokens (bw*d*esize contiguous bytes), so every
// wavefront load touches whole 256-byte-or-longer segments. The gather can
// also sum the block's real rows into its mean (the block-level features that
// selection scores), so that pooling needs no second pass over Q and K.
#include "kernels.hpp"

namespace bsa {
namespace {

struct PtrPack {
  const uint4* src[4];
  uint4* dst[4];
};

// Block means of the first n gathered tensors, fp64 [heads, M, d] each.
struct PoolPack {
  double* out[4];
  int n;
};

// Pre-attention transform of the first n gathered tensors (Q and K): RMSNorm
// over the head channels with a per-channel weight, then the 3-D rotary
// embedding. Helios page (suanlab.com, Helios review), core contributions:
// fused normalization and RoPE kernels; Kaleido page (gist.science, paper
// 2607.13770), methodology: the rotary embedding splits a head's channels
// into a time group and two spatial groups with their own frequencies.
// Reading implemented: groups t, h, w of d - 4 floor(d/6), 2 floor(d/6) and
// 2 floor(d/6) channels; pair (2i, 2i+1) of a group of g channels turns by
// pos * base^(-2i/g), pos the token's coordinate on the group's axis.
struct NormRope {
  const float* gamma[4];  // per tensor: [d] channel weights, or null (all 1)
  float eps;
  float log2_base;
  int n;
};

// The raster token of slot r of box x (-1 for a pad slot) and the slot's
// coordinates (t, h, w) on the padded grid.
__device__ inline long long slot_token_at(const Lay& L, const Box& x, int r, int& tt, int& hh,
                                          int& ww) {
  const int rw = r % x.bw;
  const int rh = (r / x.bw) % x.bh;
  const int rt = r / (x.bw * x.bh);
  tt = x.t0 + rt;
  hh = x.h0 + rh;
  ww = x.w0 + rw;
  if (rt >= x.vt || rh >= x.vh || rw >= x.vw) return -1;
  return ((long long)tt * L.H + hh) * L.W + ww;
}

constexpr int kPermThreads = 256;

// kEpc (gather only; elements per 16-byte chunk: 8 for bf16, 4 for fp32, 0 for
// a plain copy) enables the two optional stages of the gather: the
// pre-attention transform (kNR, tensors t < nr.n) and pooling (tensors
// t < pool.n): the workgroup sums the real rows of its block in fp64, from the
// values it stores, and writes the block mean. A lane keeps one chunk column
// (256 is a multiple of the chunk count), so the chunks of a row sit in
// adjacent lanes (the row's sum of squares is a shuffle reduction) and a
// lane's partial block sums need one LDS reduction over its column.
// kChunks: the row's 16-byte chunk count when it is known at compile time (16
// for bf16 and 32 for fp32 rows of d = 128), else 0 and `chunks_rt` gives it.
// The instantiations of the five uses (the Q/K/V gather with pooling, the
// pooling of Q and K alone, the plain gather, the bf16 scatter of O and the
// fp32 scatter of gradients) are distinct kernels, so per-kernel counters and
// traces tell them apart.
// kStore = false: pooling only (no dst); then a thread's loads are all issued
// before any of them is used (with stores, one chunk at a time measured
// faster: the batched form needs more registers per lane).
template <bool kInverse, int kEpc, bool kNR, int kChunks, bool kStore = true>
__global__ __launch_bounds__(kPermThreads) void permute_kernel(Lay L, const int32_t* zone_shape,
                                                               PtrPack P, int chunks_rt,
                                                               PoolPack pool, NormRope nr) {
  const int chunks = kChunks > 0 ? kChunks : chunks_rt;
  const int b = blockIdx.x;
  const int h = blockIdx.y;
  const int t = blockIdx.z;
  const Box x = block_box(L, zone_shape, b);
  const long long raster0 = (long long)h * L.N * chunks;
  const long long padded0 = ((long long)h * L.Np + (long long)b * L.B) * chunks;
  const uint4* __restrict__ src = P.src[t];
  uint4* __restrict__ dst = P.dst[t];
  const int total = L.B * chunks;  // chunks = 16-byte chunks per row
  constexpr int kAcc = kEpc > 0 ? kEpc : 1;
  double acc[kAcc];
#pragma unroll
  for (int e = 0; e < kAcc; ++e) acc[e] = 0.0;
  const bool pooled = kEpc > 0 && t < pool.n;   // uniform over the workgroup
  const bool transformed = kNR && t < nr.n;     // uniform over the workgroup

  // this lane's chunk column: channel weights and, per channel pair, the
  // rotation axis and rate (revolutions per unit of position)
  const int d = chunks * kAcc;
  const int lc = threadIdx.x & (chunks - 1);
  float gam[kAcc];
  float rate[kAcc / 2 > 0 ? kAcc / 2 : 1];
  int axis[kAcc / 2 > 0 ? kAcc / 2 : 1];
  if (kNR && transformed) {
    const float* g = nr.gamma[t];
#pragma unroll
    for (int k = 0; k < kAcc; ++k) gam[k] = g ? g[lc * kAcc + k] : 1.f;
    const int dh = 2 * (d / 6), dt = d - 2 * dh;
#pragma unroll
    for (int p = 0; p < kAcc / 2; ++p) {
      const int ch = lc * kAcc + 2 * p;
      int i, gsz;
      if (ch < dt) {
        axis[p] = 0, i = ch / 2, gsz = dt;
      } else if (ch < dt + dh) {
        axis[p] = 1, i = (ch - dt) / 2, gsz = dh;
      } else {
        axis[p] = 2, i = (ch - dt - dh) / 2, gsz = dh;
      }
      rate[p] = exp2f(-(2.f * i / gsz) * nr.log2_base) * 0.15915494309189535f;  // / 2 pi
    }
  }

  if (!kStore) {
    // pooling only: a thread's chunks (8 for a 128-slot block of bf16 d = 128
    // rows) are all requested before any is summed, so that their round trips
    // to memory overlap
    constexpr int kU = 8;
    for (int e0 = threadIdx.x; e0 < total; e0 += kU * kPermThreads) {
      uint4 vv[kU];
      bool real[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int e = e0 + u * kPermThreads;
        const int r = e / chunks;
        const long long n = e < total ? slot_token(L, x, r) : -1;
        real[u] = n >= 0;
        vv[u] = real[u] ? src[raster0 + n * chunks + (e - r * chunks)] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (!real[u]) continue;
        const uint32_t wv[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
#pragma unroll
        for (int k = 0; k < kAcc; ++k)
          acc[k] += (double)(kEpc == 8 ? __uint_as_float((k & 1) ? (wv[k >> 1] & 0xffff0000u)
                                                                  : (wv[k >> 1] << 16))
                                       : __uint_as_float(wv[k]));
      }
    }
  } else {
    for (int e = threadIdx.x; e < total; e += kPermThreads) {
      const int r = e / chunks;
      const int c = e - r * chunks;
      int tt = 0, hh = 0, ww = 0;
      const long long n = kNR ? slot_token_at(L, x, r, tt, hh, ww) : slot_token(L, x, r);
      if (!kInverse) {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (n >= 0) v = src[raster0 + n * chunks + c];
        if (kNR && transformed) {
          const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
          float f[kAcc];
  #pragma unroll
          for (int k = 0; k < kAcc; ++k)
            f[k] = kEpc == 8 ? __uint_as_float((k & 1) ? (wv[k >> 1] & 0xffff0000u) : (wv[k >> 1] << 16))
                             : __uint_as_float(wv[k]);
          // RMSNorm: the row's chunks are the `chunks` adjacent lanes
          float ss = 0.f;
  #pragma unroll
          for (int k = 0; k < kAcc; ++k) ss = fmaf(f[k], f[k], ss);
          for (int o = chunks >> 1; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
          const float inv = rsqrtf(ss / (float)d + nr.eps);
  #pragma unroll
          for (int k = 0; k < kAcc; ++k) f[k] *= inv * gam[k];
          // rotary embedding (pad rows are zero and stay zero)
  #pragma unroll
          for (int p = 0; p < kAcc / 2; ++p) {
            const int pos = axis[p] == 0 ? tt : axis[p] == 1 ? hh : ww;
            float rev = (float)pos * rate[p];
            rev -= floorf(rev);
            const float sn = __builtin_amdgcn_sinf(rev), cs = __builtin_amdgcn_cosf(rev);
            const float a0 = f[2 * p], a1 = f[2 * p + 1];
            f[2 * p] = a0 * cs - a1 * sn;
            f[2 * p + 1] = a0 * sn + a1 * cs;
          }
          uint32_t ov[4];
          if (kEpc == 8) {
            typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  #pragma unroll
            for (int k = 0; k < 4; ++k)
              ov[k] = __builtin_bit_cast(uint32_t, bf16x2v{(__bf16)f[2 * k], (__bf16)f[2 * k + 1]});
          } else {
  #pragma unroll
            for (int k = 0; k < 4; ++k) ov[k] = __float_as_uint(f[k]);
          }
          v = make_uint4(ov[0], ov[1], ov[2], ov[3]);
        }
        if (dst) dst[padded0 + e] = v;  // (no dst: pooled only)
        if (kEpc > 0 && pooled && n >= 0) {
          const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
  #pragma unroll
          for (int k = 0; k < kAcc; ++k) {
            float f;
            if (kEpc == 8)  // two bf16 per word, element 2i in the low half
              f = __uint_as_float((k & 1) ? (wv[k >> 1] & 0xffff0000u) : (wv[k >> 1] << 16));
            else
              f = __uint_as_float(wv[k]);
            acc[k] += (double)f;
          }
        }
      } else if (n >= 0) {
        dst[raster0 + n * chunks + c] = src[padded0 + e];
      }
    }
  }
  if (kEpc > 0 && pooled) {
    __shared__ double red[kPermThreads * kAcc];
#pragma unroll
    for (int k = 0; k < kAcc; ++k) red[threadIdx.x * kAcc + k] = acc[k];
    __syncthreads();
    const int groups = kPermThreads / chunks;
    for (int el = threadIdx.x; el < d; el += kPermThreads) {
      const int c = el / kAcc, k = el - c * kAcc;
      double sum = 0.0;
      for (int g = 0; g < groups; ++g) sum += red[(g * chunks + c) * kAcc + k];
      const int cnt = x.count();
      pool.out[t][((size_t)h * L.M + b) * d + el] = cnt ? sum / (double)cnt : 0.0;
    }
  }
}

// One workgroup of two wavefronts per block: wavefront v evaluates slots
// 64v .. 64v + 63, one per lane, and a ballot forms the two validity words.
// The spare words carry the block's origin as a raster token index on the
// padded grid, (t0 H + h0) W + w0, and its shape id, for kernels that read the
// block's rows straight from the token-order tensors.
__global__ __launch_bounds__(128) void block_meta_kernel(Lay L, const int32_t* zone_shape,
                                                         BlockMeta* meta) {
  const int b = blockIdx.x, r = threadIdx.x, v = r >> 6;
  const Box x = block_box(L, zone_shape, b);
  const bool real = r < L.B && slot_real(x, r);
  const uint64_t word = __ballot(real);
  if ((r & 63) == 0) {
    const uint32_t count = (uint32_t)x.count();
    uint32_t* half = meta[b].half[v];
    half[0] = (uint32_t)word;
    half[1] = (uint32_t)(word >> 32);
    half[2] = count;
    half[3] = v == 0 ? (uint32_t)(((long long)x.t0 * L.H + x.h0) * L.W + x.w0)
                     : (uint32_t)shape_id(L, zone_shape, b);
  }
}

}  // namespace

hipError_t launch_block_meta(const Lay& L, const int32_t* zone_shape, BlockMeta* meta,
                             hipStream_t st) {
  block_meta_kernel<<<L.M, 128, 0, st>>>(L, zone_shape, meta);
  return hipGetLastError();
}

hipError_t launch_permute(const Lay& L, const int32_t* zone_shape, int ntensors,
                          const void* const* src, void* const* dst, int heads, int row_bytes,
                          bool inverse, hipStream_t st, int npool, double* const* pooled,
                          int epc, int nrope, const float* const* gamma, float eps,
                          float rope_base) {
  PtrPack P{};
  for (int i = 0; i < ntensors; ++i) {
    P.src[i] = static_cast<const uint4*>(src[i]);
    P.dst[i] = static_cast<uint4*>(dst[i]);
  }
  PoolPack Q{};
  Q.n = npool;
  for (int i = 0; i < npool; ++i) Q.out[i] = pooled[i];
  NormRope R{};
  R.n = nrope;
  R.eps = eps;
  R.log2_base = nrope > 0 ? log2f(rope_base) : 0.f;
  for (int i = 0; i < nrope; ++i) R.gamma[i] = gamma ? gamma[i] : nullptr;
  const int chunks = row_bytes / 16;
  dim3 grid(L.M, heads, ntensors);
#define BSA_PERMUTE(INV, EPC, NR, CH) \
  permute_kernel<INV, EPC, NR, CH><<<grid, kPermThreads, 0, st>>>(L, zone_shape, P, chunks, Q, R)
#define BSA_POOL_ONLY(EPC, CH) \
  permute_kernel<false, EPC, false, CH, false><<<grid, kPermThreads, 0, st>>>(L, zone_shape, P, \
                                                                            chunks, Q, R)
#define BSA_PERMUTE_ROWS(INV, EPC, NR) \
  do {                                 \
    if (chunks == 16)                  \
      BSA_PERMUTE(INV, EPC, NR, 16);   \
    else if (chunks == 32)             \
      BSA_PERMUTE(INV, EPC, NR, 32);   \
    else                               \
      BSA_PERMUTE(INV, EPC, NR, 0);    \
  } while (0)
  bool pool_only = !inverse && nrope == 0 && npool == ntensors && (epc == 8 || epc == 4);
  for (int i = 0; i < ntensors; ++i) pool_only = pool_only && dst[i] == nullptr;
  if (inverse)
    BSA_PERMUTE_ROWS(true, 0, false);
  else if (pool_only && epc == 8 && chunks == 16)
    BSA_POOL_ONLY(8, 16);
  else if (pool_only && epc == 8)
    BSA_POOL_ONLY(8, 0);
  else if (pool_only)
    BSA_POOL_ONLY(4, 0);
  else if (npool == 0 && nrope == 0)
    BSA_PERMUTE_ROWS(false, 0, false);
  else if (nrope == 0 && epc == 8)
    BSA_PERMUTE(false, 8, false, 0);
  else if (nrope == 0 && epc == 4)
    BSA_PERMUTE(false, 4, false, 0);
  else if (epc == 8)
    BSA_PERMUTE(false, 8, true, 0);
  else if (epc == 4)
    BSA_PERMUTE(false, 4, true, 0);
  else
    return hipErrorInvalidValue;
#undef BSA_PERMUTE_ROWS
#undef BSA_POOL_ONLY
#undef BSA_PERMUTE
  return hipGetLastError();
}

}  // namespace bsa

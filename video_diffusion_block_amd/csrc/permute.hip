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

constexpr int kPermThreads = 256;

// kEpc > 0 (gather only): the workgroup also sums the real rows of its block
// (kEpc elements per 16-byte chunk: 8 for bf16, 4 for fp32) in fp64 and writes
// the block mean, for tensors t < pool.n. Each lane keeps one chunk column
// (256 is a multiple of the chunk count), so its partial sums need one LDS
// reduction over the lanes of that column.
template <bool kInverse, int kEpc>
__global__ __launch_bounds__(kPermThreads) void permute_kernel(Lay L, const int32_t* zone_shape,
                                                               PtrPack P, int chunks,
                                                               PoolPack pool) {
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
  const bool pooled = kEpc > 0 && t < pool.n;  // uniform over the workgroup
  for (int e = threadIdx.x; e < total; e += kPermThreads) {
    const int r = e / chunks;
    const int c = e - r * chunks;
    const long long n = slot_token(L, x, r);
    if (!kInverse) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (n >= 0) v = src[raster0 + n * chunks + c];
      dst[padded0 + e] = v;
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
  if (kEpc > 0 && pooled) {
    __shared__ double red[kPermThreads * kAcc];
#pragma unroll
    for (int k = 0; k < kAcc; ++k) red[threadIdx.x * kAcc + k] = acc[k];
    __syncthreads();
    const int d = chunks * kEpc;
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
    half[3] = 0u;
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
                          int pool_epc) {
  PtrPack P{};
  for (int i = 0; i < ntensors; ++i) {
    P.src[i] = static_cast<const uint4*>(src[i]);
    P.dst[i] = static_cast<uint4*>(dst[i]);
  }
  PoolPack Q{};
  Q.n = npool;
  for (int i = 0; i < npool; ++i) Q.out[i] = pooled[i];
  const int chunks = row_bytes / 16;
  dim3 grid(L.M, heads, ntensors);
  if (inverse)
    permute_kernel<true, 0><<<grid, kPermThreads, 0, st>>>(L, zone_shape, P, chunks, Q);
  else if (npool == 0)
    permute_kernel<false, 0><<<grid, kPermThreads, 0, st>>>(L, zone_shape, P, chunks, Q);
  else if (pool_epc == 8)
    permute_kernel<false, 8><<<grid, kPermThreads, 0, st>>>(L, zone_shape, P, chunks, Q);
  else if (pool_epc == 4)
    permute_kernel<false, 4><<<grid, kPermThreads, 0, st>>>(L, zone_shape, P, chunks, Q);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace bsa

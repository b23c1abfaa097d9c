// Token <-> block-order gather/scatter.
//
// Prism page (trawling.dev/post/2299), section on block composition matched to
// regional information: tokens of a macro-zone are regrouped into blocks of the
// zone's shape. One workgroup moves one (block, head, tensor) tile: B rows of
// d elements, 16 bytes per lane per step. Source rows of a block come in runs
// of bw consecutive raster tokens (bw*d*esize contiguous bytes), so every
// wavefront load touches whole 256-byte-or-longer segments.
#include "kernels.hpp"

namespace bsa {
namespace {

struct PtrPack {
  const uint4* src[4];
  uint4* dst[4];
};

constexpr int kPermThreads = 256;

template <bool kInverse>
__global__ __launch_bounds__(kPermThreads) void permute_kernel(Lay L, const int32_t* zone_shape,
                                                               PtrPack P, int chunks) {
  const int b = blockIdx.x;
  const int h = blockIdx.y;
  const int t = blockIdx.z;
  const Box x = block_box(L, zone_shape, b);
  const long long raster0 = (long long)h * L.N * chunks;
  const long long padded0 = ((long long)h * L.Np + (long long)b * L.B) * chunks;
  const uint4* __restrict__ src = P.src[t];
  uint4* __restrict__ dst = P.dst[t];
  const int total = L.B * chunks;  // chunks = 16-byte chunks per row
  for (int e = threadIdx.x; e < total; e += kPermThreads) {
    const int r = e / chunks;
    const int c = e - r * chunks;
    const long long n = slot_token(L, x, r);
    if (!kInverse) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (n >= 0) v = src[raster0 + n * chunks + c];
      dst[padded0 + e] = v;
    } else if (n >= 0) {
      dst[raster0 + n * chunks + c] = src[padded0 + e];
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
                          bool inverse, hipStream_t st) {
  PtrPack P{};
  for (int i = 0; i < ntensors; ++i) {
    P.src[i] = static_cast<const uint4*>(src[i]);
    P.dst[i] = static_cast<uint4*>(dst[i]);
  }
  const int chunks = row_bytes / 16;
  dim3 grid(L.M, heads, ntensors);
  if (inverse)
    permute_kernel<true><<<grid, kPermThreads, 0, st>>>(L, zone_shape, P, chunks);
  else
    permute_kernel<false><<<grid, kPermThreads, 0, st>>>(L, zone_shape, P, chunks);
  return hipGetLastError();
}

}  // namespace bsa

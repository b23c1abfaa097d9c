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

__global__ __launch_bounds__(256) void block_meta_kernel(Lay L, const int32_t* zone_shape,
                                                         BlockMeta* meta) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= L.M) return;
  const Box x = block_box(L, zone_shape, b);
  uint32_t words[4] = {0u, 0u, 0u, 0u};
  for (int r = 0; r < L.B && r < 128; ++r)
    if (slot_real(x, r)) words[r >> 5] |= 1u << (r & 31);
  BlockMeta m;
  for (int h = 0; h < 2; ++h) {
    m.half[h][0] = words[2 * h];
    m.half[h][1] = words[2 * h + 1];
    m.half[h][2] = (uint32_t)x.count();
    m.half[h][3] = 0u;
  }
  meta[b] = m;
}

}  // namespace

hipError_t launch_block_meta(const Lay& L, const int32_t* zone_shape, BlockMeta* meta,
                             hipStream_t st) {
  block_meta_kernel<<<(L.M + 255) / 256, 256, 0, st>>>(L, zone_shape, meta);
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

// Token layout arithmetic shared by the host validation and the HIP kernels.
//
// Macro-zones and per-zone block shapes follow the Prism page
// (trawling.dev/post/2299, section on block composition matched to regional
// information): tokens are partitioned into spatio-temporal macro-zones and
// each zone is cut into blocks of its own shape. The order used here: zones
// raster over the zone grid, blocks raster inside a zone, tokens raster inside
// a block; every axis padded up to a multiple of the zone extent.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

struct Lay {
  int T, H, W;        // latent grid
  int zt, zh, zw;     // zone extent
  int gzt, gzh, gzw;  // zone grid
  int n_shapes;
  int sh[4][3];       // candidate block shapes (bt, bh, bw)
  int B;              // tokens per block
  int bpz;            // blocks per zone
  int M;              // blocks
  int nZ;             // zones
  long long N;        // real tokens
  long long Np;       // padded slots = M * B
};

// Box of block b: origin (t0,h0,w0) in the padded grid, shape (bt,bh,bw) and
// the number of real rows along each axis (vt,vh,vw), possibly 0.
struct Box {
  int t0, h0, w0;
  int bt, bh, bw;
  int vt, vh, vw;
  __host__ __device__ int count() const { return vt * vh * vw; }
};

__host__ __device__ inline int imin(int a, int b) { return a < b ? a : b; }
__host__ __device__ inline int imax(int a, int b) { return a > b ? a : b; }

// Shape id of block b's zone (ids come from device memory; an out-of-range id
// is clamped).
__host__ __device__ inline int shape_id(const Lay& L, const int32_t* zone_shape, int b) {
  return zone_shape ? imin(imax(zone_shape[b / L.bpz], 0), L.n_shapes - 1) : 0;
}

__host__ __device__ inline Box block_box(const Lay& L, const int32_t* zone_shape, int b) {
  const int z = b / L.bpz;
  const int local = b - z * L.bpz;
  const int s = shape_id(L, zone_shape, b);
  Box x;
  x.bt = L.sh[s][0];
  x.bh = L.sh[s][1];
  x.bw = L.sh[s][2];
  const int nh = L.zh / x.bh, nw = L.zw / x.bw;
  const int lt = local / (nh * nw), lh = (local / nw) % nh, lw = local % nw;
  const int zzt = z / (L.gzh * L.gzw), zzh = (z / L.gzw) % L.gzh, zzw = z % L.gzw;
  x.t0 = zzt * L.zt + lt * x.bt;
  x.h0 = zzh * L.zh + lh * x.bh;
  x.w0 = zzw * L.zw + lw * x.bw;
  x.vt = imax(0, imin(x.bt, L.T - x.t0));
  x.vh = imax(0, imin(x.bh, L.H - x.h0));
  x.vw = imax(0, imin(x.bw, L.W - x.w0));
  return x;
}

// Raster token id of slot r (0 <= r < B) of a block, or -1 for a pad slot.
__host__ __device__ inline long long slot_token(const Lay& L, const Box& x, int r) {
  const int rw = r % x.bw;
  const int rh = (r / x.bw) % x.bh;
  const int rt = r / (x.bw * x.bh);
  if (rt >= x.vt || rh >= x.vh || rw >= x.vw) return -1;
  return ((long long)(x.t0 + rt) * L.H + (x.h0 + rh)) * L.W + (x.w0 + rw);
}

__host__ __device__ inline bool slot_real(const Box& x, int r) {
  const int rw = r % x.bw;
  const int rh = (r / x.bw) % x.bh;
  const int rt = r / (x.bw * x.bh);
  return rt < x.vt && rh < x.vh && rw < x.vw;
}

}  // namespace bsa

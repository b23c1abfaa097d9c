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
#include "bsa.h"
#include "kernels.hpp"

namespace bsa {
namespace {

// ------------------------------------------------------ D = rowsum(dO * O) --
// G = d / (elements per 16 bytes) lanes per row (8, 16 or 32), one 16-byte
// chunk of O and dO each; the row sum is a shuffle reduction inside the group.
// Also writes lse2 = lse log2(e), the row's lse in the units of the matrix
// kernels' base-2 exponentials (one multiply per row instead of one per score).
template <typename T>
__global__ __launch_bounds__(256) void delta_kernel(const T* op, const T* dop, const float* lse,
                                                    int d, long long rows, float* delta,
                                                    float* lse2) {
  constexpr int EPC = 16 / sizeof(T);
  const int G = d / EPC;
  const long long r = ((long long)blockIdx.x * 256 + threadIdx.x) / G;
  const int c = threadIdx.x % G;
  const bool ok = r < rows;
  const size_t base = (size_t)(ok ? r : 0) * d + (size_t)c * EPC;
  float acc = 0.f;
  if constexpr (sizeof(T) == 2) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(op + base);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(dop + base);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += (float)a[i] * (float)b[i];
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(op + base);
    const f32x4 b = *reinterpret_cast<const f32x4*>(dop + base);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += a[i] * b[i];
  }
  for (int off = G / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (ok && c == 0) {
    delta[r] = acc;
    lse2[r] = lse[r] * kLog2e;
  }
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

// The key blocks of head h by decreasing key-major list length (equal lengths
// in any order): order[h * M + r] is the r-th longest. The dK/dV pass takes
// its workgroups in this order. Its work per key block grows with the list
// length (0 for pad blocks, up to several hundred listed query blocks), and
// with the longest lists started first the short ones fill in the last wave
// of workgroups instead of one long list running on alone. The outputs do not
// depend on the order. A counting sort: lengths histogram, exclusive scan from
// the longest length down, then each block takes the next slot of its length.
__global__ __launch_bounds__(1024) void longest_first_kernel(Lay L, const int32_t* tcounts,
                                                             int32_t* order) {
  __shared__ int slot[BSA_MAX_BLOCKS + 1];  // per length: count, then next free rank
  __shared__ int part[1024];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int nl = L.M + 1;  // lengths 0..M
  const int32_t* len = tcounts + (size_t)h * L.M;
  for (int b = tid; b < nl; b += 1024) slot[b] = 0;
  __syncthreads();
  for (int j = tid; j < L.M; j += 1024) atomicAdd(&slot[min(max(len[j], 0), L.M)], 1);
  __syncthreads();
  // thread t owns the lengths M - t*S .. M - t*S - S + 1 (longest first)
  const int S = (nl + 1023) / 1024;
  int own = 0;
  for (int s = 0; s < S; ++s) {
    const int r = tid * S + s;
    if (r < nl) own += slot[L.M - r];
  }
  part[tid] = own;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int rank = part[tid] - own;  // blocks longer than this thread's lengths
  for (int s = 0; s < S; ++s) {
    const int r = tid * S + s;
    if (r < nl) {
      const int c = slot[L.M - r];
      slot[L.M - r] = rank;
      rank += c;
    }
  }
  __syncthreads();
  for (int j = tid; j < L.M; j += 1024)
    order[(size_t)h * L.M + atomicAdd(&slot[min(max(len[j], 0), L.M)], 1)] = j;
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

// ------------------------------------------------------------- MFMA path --
// bf16, d = 128, 128-token blocks. Tiles live in LDS row-major (256-byte rows of
// 16 chunks) with the chunk swizzle q ^ (4 (r & 3) + ((r >> 2) & 3)), which is
// bank-conflict free both for row reads (16 consecutive rows, one chunk) and
// for the gfx950 transposing reads (4 consecutive rows x 4 chunks).
constexpr int kD = 128;
constexpr int kB = 128;
constexpr int kTile = kB * kD;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

__device__ inline int uswz_f(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

__device__ inline bf16x4 tr_read(const __bf16* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// Direct global->LDS copy of one 128 x 128 bf16 tile by kWaves wavefronts:
// load m of wave w fills LDS slots (kWaves m + w) * 64 + lane (row r = slot/16,
// physical chunk lane % 16), fetching the logical chunk the swizzle puts there.
template <int kWaves>
__device__ inline void dma_tile(__bf16* tile, const __bf16* gtile, int w, int lane) {
#pragma unroll
  for (int m = 0; m < 32 / kWaves; ++m) {
    const int r = 4 * (kWaves * m + w) + (lane >> 4);
    const int q = (lane & 15) ^ uswz_f(r);
    __builtin_amdgcn_global_load_lds(gtile + r * kD + 8 * q,
                                     (lds_void*)(tile + (kWaves * m + w) * 512), 16, 0, 0);
  }
}

// Offsets (bf16 elements) of the two transposed reads that give lane
// (G = lane/16, u = lane%16) the A operand rows [R + 0..3] and [R + 8..11] of
// column 32t + l32, R = base row + 16c + 4hi (add 16c*kD for k-step c).
__device__ inline void tr_offsets(int (&o1)[4], int (&o2)[4], int row0, int lane) {
  const int G = lane >> 4, u = lane & 15, hi = lane >> 5;
  const int vy = u >> 2, vx = 2 * (G & 1) + ((u & 3) >> 1);
  const int r1 = row0 + 4 * hi + vy, r2 = r1 + 8;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    o1[t] = r1 * kD + 8 * ((4 * t + vx) ^ uswz_f(r1)) + 4 * (u & 1);
    o2[t] = r2 * kD + 8 * ((4 * t + vx) ^ uswz_f(r2)) + 4 * (u & 1);
  }
}

// dQ for one (query block, head): for every listed key block j,
//   S^T = K Q^T, dP^T = V dO^T, P^T = exp(S^T scale - lse), dS^T = P^T (dP^T - D),
//   dQ^T += K^T dS^T  (K^T through transposed LDS reads).
// 8 wavefronts: wave w owns queries 32 (w % 4) .. +32 and keys 64 (w / 4) .. +64.
// Raster token of slot r of a block, from its table entry (origin, shape); r
// must be a real slot. The entry is read at a uniform index, so L.sh[shape]
// is a scalar load.
__device__ inline long long slot_raster(const Lay& L, const BlockMeta& m, int r) {
  const int s = __builtin_amdgcn_readfirstlane(m.shape());
  const int bw = L.sh[s][2], bh = L.sh[s][1];
  return (long long)m.origin() + ((r / (bw * bh)) * L.H + (r / bw) % bh) * L.W + r % bw;
}

__global__ __launch_bounds__(512, 1) void attn_bwd_dq_mfma(
    Lay L, const BlockMeta* __restrict__ meta, const __bf16* __restrict__ qp,
    const __bf16* __restrict__ kp, const __bf16* __restrict__ vp,
    const __bf16* __restrict__ dop, const float* __restrict__ lse2,
    const float* __restrict__ delta, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ idx, float scale, float* __restrict__ dqp, int raster) {
  __shared__ __align__(16) __bf16 sK[2][kTile];
  __shared__ __align__(16) __bf16 sV[2][kTile];
  __shared__ int32_t sList[BSA_MAX_BLOCKS];      // the row's key-block list
  __shared__ __align__(16) uint32_t sM[2][64];   // block facts of the current/next block
  const int i = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qg = w & 3, kh = w >> 2;
  const int l32 = lane & 31, hi = lane >> 5;
  const size_t row = (size_t)h * L.M + i;
  const int n = counts[row];
  const int32_t* lst = idx + row * L.M;
  const size_t head0 = (size_t)h * L.Np;
  const int q = 32 * qg + l32;
  const bool q_real = (meta[i].mask(q >> 5) >> (q & 31)) & 1u;
  // the lane's row of the block-ordered inputs, and its dQ row: the same slot
  // of [H, Np, d], or (raster) its token's row of [H, N, d] (pad slots there
  // have no row and write nothing)
  const size_t qrow = head0 + (size_t)i * kB + q;
  const size_t orow =
      raster ? (size_t)h * L.N + (size_t)(q_real ? slot_raster(L, meta[i], q) : 0) : qrow;
  const bool q_write = q_real || !raster;

  if (n == 0) {
    if (kh == 0 && q_write)
      for (int e = 8 * hi; e < kD; e += 16)
        *reinterpret_cast<f32x4*>(dqp + orow * kD + e) = f32x4{0.f, 0.f, 0.f, 0.f},
        *reinterpret_cast<f32x4*>(dqp + orow * kD + e + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  const uint32_t head_bytes = (uint32_t)L.Np * kD * 2;
  const i32x4 krs = make_buffer_rsrc(kp + head0 * kD, head_bytes);
  const i32x4 vrs = make_buffer_rsrc(vp + head0 * kD, head_bytes);
  const i32x4 mrs = make_buffer_rsrc(meta, (uint32_t)L.M * sizeof(BlockMeta));
  // tile load m (0..3) of wave w: LDS slots (8m + w) * 64 + lane (swizzled fetch)
  auto dma_part = [&](__bf16* tile, const i32x4& rs, int src, int m) {
    const int r = 4 * (8 * m + w) + (lane >> 4);
    const int qq = (lane & 15) ^ uswz_f(r);
    dma16_manual(rs, lds_addr_of(tile + (8 * m + w) * 512), 2 * (r * kD + 8 * qq), src);
  };
  // block blk's 32-byte record into slot sM[slot] (wave 0, one dword per lane)
  auto fetch_meta = [&](int blk, int slot) {
    if (w == 0) dma4_manual(mrs, lds_addr_of(&sM[slot][0]), 4 * (lane & 7), blk * 32);
  };
  for (int e = tid; e < n; e += 512) sList[e] = lst[e];
  {
    const int b0 = lst[0];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      dma_part(sK[0], krs, b0 * kTile * 2, m);
      dma_part(sV[0], vrs, b0 * kTile * 2, m);
    }
    fetch_meta(b0, 0);
  }

  bf16x8 qf[8], dof[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    qf[s] = *reinterpret_cast<const bf16x8*>(qp + qrow * kD + 16 * s + 8 * hi);
    dof[s] = *reinterpret_cast<const bf16x8*>(dop + qrow * kD + 16 * s + 8 * hi);
  }
  const float c2 = scale * kLog2e;
  const float lq2 = lse2[qrow];
  const float dq_d = delta[qrow];
  const bf16x8 bias_b = pad_bias_b(hi);

  const int rowA = 64 * kh + l32;          // row-read operand rows (+32 kt)
  const int fA = uswz_f(l32);
  int o1[4], o2[4];
  tr_offsets(o1, o2, 64 * kh, lane);

  f32x16 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  asm volatile("" ::"s"(c2));
  __builtin_amdgcn_s_waitcnt(0);  // everything, the hand-issued loads included
  __syncthreads();

  for (int jj = 0; jj < n; ++jj) {
    const int b = jj & 1;
    const bool more = jj + 1 < n;
    const int bn = more ? __builtin_amdgcn_readfirstlane(sList[jj + 1]) : 0;
    // this block's validity words (this wave's 64 keys) and real-slot count
    const uint32_t mw0 = sM[b][4 * kh], mw1 = sM[b][4 * kh + 1];
    const bool partial = __builtin_amdgcn_readfirstlane((int)sM[b][2]) < kB;
    const __bf16* sk = sK[b];
    const __bf16* sv = sV[b];
    f32x16 st[2], dpt[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      // the next block's tiles and facts, spread over the products
      if (more) {
        dma_part(sK[b ^ 1], krs, bn * kTile * 2, 2 * kt);
        dma_part(sK[b ^ 1], krs, bn * kTile * 2, 2 * kt + 1);
        if (kt == 0) fetch_meta(bn, b ^ 1);
      }
      const int ro = (rowA + 32 * kt) * kD;
      bf16x8 fa[8], fb[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int off = ro + 8 * ((2 * s + hi) ^ fA);
        fa[s] = *reinterpret_cast<const bf16x8*>(sk + off);
        fb[s] = *reinterpret_cast<const bf16x8*>(sv + off);
      }
      // k-step 0 from an immediate zero accumulator (no register clearing);
      // a partial block's pad keys get the -2^30 bias product last (it adds
      // an exact 0 to every real key's score)
      const f32x16 zero = {};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        st[kt] = mfma32x32x16(fa[s], qf[s], s == 0 ? zero : st[kt]);
        dpt[kt] = mfma32x32x16(fb[s], dof[s], s == 0 ? zero : dpt[kt]);
      }
      if (partial) st[kt] = mfma32x32x16(pad_bias_a(kt ? mw1 : mw0, l32, hi), bias_b, st[kt]);
    }
    bf16x8 dsf[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_fast(fmaf(st[kt][r], c2, -lq2));  // 0 for pad keys
        dsf[2 * kt + (r >> 3)][r & 7] = (__bf16)(p * (dpt[kt][r] - dq_d));
      }
    }
    // dQ^T (d x queries) += K^T (d x keys) dS^T (keys x queries)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (more) dma_part(sV[b ^ 1], vrs, bn * kTile * 2, t);
      bf16x8 a[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x4 lo = tr_read(sk + o1[t] + 16 * c * kD);
        const bf16x4 up = tr_read(sk + o2[t] + 16 * c * kD);
        a[c] = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[t] = mfma32x32x16(a[c], dsf[c], acc[t]);
    }
    // the next block's tiles and facts have landed (every wave its own part)
    // before anyone reads them; this block's buffers are free after the barrier
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    asm volatile("s_barrier" ::: "memory");
  }
  // sum the two key halves (waves w and w+4 share their 32 queries)
  // element e of lane (qg, lane) at xo[256 e]: conflict-free accesses
  float* xo = reinterpret_cast<float*>(&sK[0][0]) + qg * 64 + lane;
  if (kh == 1) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[256 * (16 * t + r)] = acc[t][r];
  }
  __syncthreads();
  if (kh == 0 && q_write) {
    float* out = dqp + orow * kD;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          v[rr] = q_real ? (acc[t][4 * g + rr] + xo[256 * (16 * t + 4 * g + rr)]) * scale : 0.f;
        *reinterpret_cast<f32x4*>(out + 32 * t + 8 * g + 4 * hi) = v;
      }
  }
}

// dK and dV for one (key block, head): for every query block i whose list
// holds the key block (key-major list),
//   S = Q K^T, dP = dO V^T, P = exp(S scale - lse), dS = P (dP - D),
//   dV += P^T dO, dK += dS^T Q   (dO and Q through transposed LDS reads).
// 4 wavefronts (one per SIMD): wave w owns keys 32w .. +32; K and V fragments
// stay in registers; Q_i, dO_i, lse_i and D_i stream through LDS. Within a
// query block the four 32-query tiles are software-pipelined: the S and dP
// products of tile qt+1 are issued before the exponentials of tile qt, so the
// matrix pipe works while the vector unit computes P and dS.
// Tile loads are issued by hand (buffer loads into LDS, see dma16_manual): the
// kernel waits for them itself (vmcnt(0) before the per-block barrier) and the
// barrier is a bare s_barrier.
constexpr int kMaxList = BSA_MAX_BLOCKS;

__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv_mfma(
    Lay L, const BlockMeta* __restrict__ meta, const __bf16* __restrict__ qp,
    const __bf16* __restrict__ kp, const __bf16* __restrict__ vp,
    const __bf16* __restrict__ dop, const float* __restrict__ lse2,
    const float* __restrict__ delta, const int32_t* __restrict__ tcounts,
    const int32_t* __restrict__ tidx, const int32_t* __restrict__ order, float scale,
    float* __restrict__ dkp, float* __restrict__ dvp, int raster) {
  __shared__ __align__(16) __bf16 sQ[2][kTile];
  __shared__ __align__(16) __bf16 sO[2][kTile];
  __shared__ __align__(16) float sL[2][kB];
  __shared__ __align__(16) float sD[2][kB];
  __shared__ int32_t sList[kMaxList];
  // workgroup x of head h takes the key block of the x-th longest list
  const int h = blockIdx.y;
  const int j = __builtin_amdgcn_readfirstlane(order[(size_t)h * L.M + blockIdx.x]);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const size_t row = (size_t)h * L.M + j;
  const int n = tcounts[row];
  const int32_t* lst = tidx + row * L.M;
  const size_t head0 = (size_t)h * L.Np;
  const size_t kbase = head0 + (size_t)j * kB;   // first slot of the key block

  f32x16 dk[4], dv[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[t][r] = dv[t][r] = 0.f;

  if (n > 0) {
    const uint32_t head_bytes = (uint32_t)L.Np * kD * 2;
    const i32x4 qrs = make_buffer_rsrc(qp + head0 * kD, head_bytes);
    const i32x4 ors = make_buffer_rsrc(dop + head0 * kD, head_bytes);
    const i32x4 lrs = make_buffer_rsrc(lse2 + head0, (uint32_t)L.Np * 4);
    const i32x4 drs = make_buffer_rsrc(delta + head0, (uint32_t)L.Np * 4);
    // tile load m (0..7) of wave w: LDS slots (4m + w) * 64 + lane, i.e. row
    // 4 (4m + w) + lane / 16, physical chunk lane % 16 (swizzled fetch)
    auto dma_part = [&](__bf16* tile, const i32x4& rs, int src, int m) {
      const int r = 4 * (4 * m + w) + (lane >> 4);
      const int q = (lane & 15) ^ uswz_f(r);
      dma16_manual(rs, lds_addr_of(tile + (4 * m + w) * 512), 2 * (r * kD + 8 * q), src);
    };
    // the 128 lse2 and delta values of query block ib (512 bytes each): waves 0, 1, lanes 0..31
    auto dma_stats = [&](int buf, int ib) {
      if (w < 2 && lane < 32)
        dma16_manual(w == 0 ? lrs : drs, lds_addr_of(w == 0 ? &sL[buf][0] : &sD[buf][0]),
                     16 * lane, ib * kB * 4);
    };
    for (int e = tid; e < n; e += 256) sList[e] = lst[e];
    {
      const int ib = lst[0];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        dma_part(sQ[0], qrs, ib * kTile * 2, m);
        dma_part(sO[0], ors, ib * kTile * 2, m);
      }
      dma_stats(0, ib);
    }

    // K and V fragments (B operands of S = Q K^T and dP = dO V^T):
    // lane holds K[key 32w + l32][16s + 8hi .. +8].
    bf16x8 kf[8], vf[8];
    const size_t krow = (kbase + 32 * w + l32) * kD + 8 * hi;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      kf[s] = *reinterpret_cast<const bf16x8*>(kp + krow + 16 * s);
      vf[s] = *reinterpret_cast<const bf16x8*>(vp + krow + 16 * s);
    }
    const float c2 = scale * kLog2e;
    const int fA = uswz_f(l32);
    int o1[4], o2[4];
    tr_offsets(o1, o2, 0, lane);
    asm volatile("" ::"s"(c2));
    __builtin_amdgcn_s_waitcnt(0);  // everything, the hand-issued loads included
    __syncthreads();

    // S and dP tiles of queries 32qt + (0..31) x keys 32w + (0..31)
    auto sdp = [&](const __bf16* sq, const __bf16* so, int qt, f32x16& sc, f32x16& dpc) {
      const int ro = (32 * qt + l32) * kD;
      bf16x8 a[8], b[8];
      auto load = [&](int s) {
        const int off = ro + 8 * ((2 * s + hi) ^ fA);
        a[s] = *reinterpret_cast<const bf16x8*>(sq + off);
        b[s] = *reinterpret_cast<const bf16x8*>(so + off);
      };
      // fragments requested four k-steps (eight products) ahead of their use
#pragma unroll
      for (int s = 0; s < 4; ++s) load(s);
      __builtin_amdgcn_sched_barrier(0);
      const f32x16 zero = {};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        sc = mfma32x32x16(a[s], kf[s], s == 0 ? zero : sc);
        dpc = mfma32x32x16(b[s], vf[s], s == 0 ? zero : dpc);
        if (s + 4 < 8) load(s + 4);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    for (int ii = 0; ii < n; ++ii) {
      const int b = ii & 1;
      const bool more = ii + 1 < n;
      const int ib1 = more ? __builtin_amdgcn_readfirstlane(sList[ii + 1]) : 0;
      const __bf16* sq = sQ[b];
      const __bf16* so = sO[b];
      f32x16 sc, dpc;
      sdp(sq, so, 0, sc, dpc);
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        // next block's tiles, two loads of each per query tile
        if (more) {
          dma_part(sQ[b ^ 1], qrs, ib1 * kTile * 2, 2 * qt);
          dma_part(sQ[b ^ 1], qrs, ib1 * kTile * 2, 2 * qt + 1);
          dma_part(sO[b ^ 1], ors, ib1 * kTile * 2, 2 * qt);
          dma_part(sO[b ^ 1], ors, ib1 * kTile * 2, 2 * qt + 1);
          if (qt == 0) dma_stats(b ^ 1, ib1);
        }
        // S and dP of the next query tile: all sixteen fragments requested
        // first, then the products interleaved one by one with the vector
        // work of this tile (a wavefront issues in order, so the matrix pipe
        // stays busy only if its instructions are spread through the VALU ones)
        f32x16 sn, dpn;
        bf16x8 na[8], nb[8];
        f32x4 l4[4], d4[4];
        const int nro = (32 * (qt + 1) + l32) * kD;
        auto nload = [&](int s) {
          const int off = nro + 8 * ((2 * s + hi) ^ fA);
          na[s] = *reinterpret_cast<const bf16x8*>(sq + off);
          nb[s] = *reinterpret_cast<const bf16x8*>(so + off);
        };
        if (qt < 3) {
#pragma unroll
          for (int s = 0; s < 4; ++s) nload(s);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          l4[g] = *reinterpret_cast<const f32x4*>(&sL[b][32 * qt + 8 * g + 4 * hi]);
          d4[g] = *reinterpret_cast<const f32x4*>(&sD[b][32 * qt + 8 * g + 4 * hi]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (qt < 3) {
          const f32x16 zero = {};
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            sn = mfma32x32x16(na[s], kf[s], s == 0 ? zero : sn);
            dpn = mfma32x32x16(nb[s], vf[s], s == 0 ? zero : dpn);
            if (s + 4 < 8) nload(s + 4);
          }
        }
        // element r belongs to query 32qt + 8(r/4) + 4hi + r%4
        bf16x8 pf[2], dsf[2];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int r = 4 * g + rr;
            const float p = exp2_fast(fmaf(sc[r], c2, -l4[g][rr]));
            pf[r >> 3][r & 7] = (__bf16)p;
            dsf[r >> 3][r & 7] = (__bf16)(p * (dpc[r] - d4[g][rr]));
          }
        }
        if (qt < 3) {
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // six VALU
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // six VALU
            if (k < 4) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        // dV (keys x d) += P^T (keys x queries) dO (queries x d), and
        // dK += dS^T Q: k-step c covers queries 32qt + 16c + ..., read transposed.
        bf16x8 ob[4][2], qb[4][2];
        auto tload = [&](int t) {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int base = (32 * qt + 16 * c) * kD;
            ob[t][c] = __builtin_shufflevector(tr_read(so + base + o1[t]),
                                               tr_read(so + base + o2[t]), 0, 1, 2, 3, 4, 5, 6, 7);
            qb[t][c] = __builtin_shufflevector(tr_read(sq + base + o1[t]),
                                               tr_read(sq + base + o2[t]), 0, 1, 2, 3, 4, 5, 6, 7);
          }
        };
        // transposed fragments requested one d-tile (four products) ahead
        tload(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (t + 1 < 4) tload(t + 1);
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            dv[t] = mfma32x32x16(pf[c], ob[t][c], dv[t]);
            dk[t] = mfma32x32x16(dsf[c], qb[t][c], dk[t]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (qt < 3) {
          sc = sn;
          dpc = dpn;
        }
      }
      // the next block's tiles have landed (every wave its own part) before
      // anyone reads them; this block's buffers are free after the barrier
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      asm volatile("s_barrier" ::: "memory");
    }
  }
  // lane holds rows key 32w + 8(r/4) + 4hi + r%4, column d = 32t + l32;
  // raster: the key's token row of [H, N, d] (pad slots have none)
  const BlockMeta& mj = meta[j];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = 32 * w + 8 * (r >> 2) + 4 * hi + (r & 3);
    const bool real = (mj.mask(key >> 5) >> (key & 31)) & 1u;
    if (raster && !real) continue;
    const size_t krow = raster ? (size_t)h * L.N + (size_t)slot_raster(L, mj, key) : kbase + key;
    float* dkr = dkp + krow * kD + l32;
    float* dvr = dvp + krow * kD + l32;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      dkr[32 * t] = real ? dk[t][r] * scale : 0.f;
      dvr[32 * t] = real ? dv[t][r] : 0.f;
    }
  }
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
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k1),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh_kv);
  if (e != hipSuccess) return e;
  k1<<<grid, L.B, sh_kv, st>>>(L, zs, q, k, v, dO, lse, delta, tcounts, tidx, scale, dk, dv);
  const size_t sh_q = 2 * (size_t)L.B * D * sizeof(float);
  auto k2 = dq_scalar<T, D>;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(k2),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh_q);
  if (e != hipSuccess) return e;
  k2<<<grid, L.B, sh_q, st>>>(L, zs, q, k, v, dO, lse, delta, counts, idx, scale, dq);
  return hipGetLastError();
}

}  // namespace

// Workspace: delta [H, Np] f32 | lse2 [H, Np] f32 | bitmap [H, M, words] u32 |
// tcounts [H, M] | tidx [H, M, M] | block table [M]
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t attn_bwd_workspace(const Lay& L, int heads, int d) {
  (void)d;
  const size_t words = (L.M + 31) / 32;
  return 2 * align256((size_t)heads * L.Np * sizeof(float)) +
         align256((size_t)heads * L.M * words * sizeof(uint32_t)) +
         align256((size_t)heads * L.M * sizeof(int32_t)) +
         align256((size_t)heads * L.M * L.M * sizeof(int32_t)) +
         align256((size_t)L.M * sizeof(BlockMeta)) +
         align256((size_t)heads * L.M * sizeof(int32_t));
}

hipError_t launch_attn_bwd(const Lay& L, const int32_t* zone_shape, const void* qp,
                           const void* kp, const void* vp, const void* op, const void* dop,
                           const float* lse, const int32_t* counts, const int32_t* idx,
                           int heads, int d, bool bf16, float scale, void* dqp, void* dkp,
                           void* dvp, void* ws, hipStream_t st, bool raster) {
  const int words = (L.M + 31) / 32;
  char* p = static_cast<char*>(ws);
  float* delta = reinterpret_cast<float*>(p);
  p += align256((size_t)heads * L.Np * sizeof(float));
  float* lse2 = reinterpret_cast<float*>(p);
  p += align256((size_t)heads * L.Np * sizeof(float));
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)heads * L.M * words * sizeof(uint32_t));
  int32_t* tcounts = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)heads * L.M * sizeof(int32_t));
  int32_t* tidx = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)heads * L.M * L.M * sizeof(int32_t));
  BlockMeta* meta = reinterpret_cast<BlockMeta*>(p);
  p += align256((size_t)L.M * sizeof(BlockMeta));
  int32_t* order = reinterpret_cast<int32_t*>(p);

  const long long rows = (long long)heads * L.Np;
  const int lanes_per_row = d * (bf16 ? 2 : 4) / 16;
  const unsigned dgrid = (unsigned)((rows * lanes_per_row + 255) / 256);
  if (bf16)
    delta_kernel<__bf16><<<dgrid, 256, 0, st>>>(static_cast<const __bf16*>(op),
                                                  static_cast<const __bf16*>(dop), lse, d, rows,
                                                  delta, lse2);
  else
    delta_kernel<float><<<dgrid, 256, 0, st>>>(static_cast<const float*>(op),
                                                 static_cast<const float*>(dop), lse, d, rows,
                                                 delta, lse2);
  bitmap_kernel<<<dim3(L.M, heads), 256, 0, st>>>(L, counts, idx, words, bitmap);
  transpose_kernel<<<dim3(L.M, heads), 256, 0, st>>>(L, bitmap, words, tcounts, tidx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  if (bf16 && d == kD && L.B == kB) {
    e = launch_block_meta(L, zone_shape, meta, st);
    if (e != hipSuccess) return e;
    longest_first_kernel<<<heads, 1024, 0, st>>>(L, tcounts, order);
    const __bf16* q = static_cast<const __bf16*>(qp);
    const __bf16* k = static_cast<const __bf16*>(kp);
    const __bf16* v = static_cast<const __bf16*>(vp);
    const __bf16* dO = static_cast<const __bf16*>(dop);
    attn_bwd_dkdv_mfma<<<dim3(L.M, heads), 256, 0, st>>>(L, meta, q, k, v, dO, lse2, delta,
                                                        tcounts, tidx, order, scale,
                                                        static_cast<float*>(dkp),
                                                        static_cast<float*>(dvp), raster ? 1 : 0);
    attn_bwd_dq_mfma<<<dim3(L.M, heads), 512, 0, st>>>(L, meta, q, k, v, dO, lse2, delta, counts,
                                                      idx, scale, static_cast<float*>(dqp),
                                                      raster ? 1 : 0);
    return hipGetLastError();
  }
  if (raster) return hipErrorInvalidValue;  // (raster gradients need the MFMA kernels)

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

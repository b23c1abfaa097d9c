// Block-sparse attention forward.
//
// Prism page (trawling.dev/post/2299), section on block composition matched to
// regional information: Prism Block Sparse Attention attends every query block
// only to its selected key blocks. For each real query slot n of block i:
//   O[n] = sum_m softmax_m(Q_n . K_m * scale) V_m over the real slots m of the
//   listed key blocks;  lse[n] = ln sum_m exp(Q_n . K_m * scale).
//
// Two kernels:
//  * attn_fwd_mfma: bf16, d = 128, 128-token blocks. One workgroup of 8
//    wavefronts per (query block, head). Wave w owns queries 32*(w%4)..+32 and
//    keys 64*(w/4)..+64 of every listed key block. S is computed transposed
//    (S^T = K Q^T on v_mfma_f32_32x32x16_bf16) so that a lane holds one query's
//    scores: the softmax row reductions stay inside the lane (plus one exchange
//    with the lane 32 away), and O^T = V^T P^T keeps the per-query rescale
//    lane-local too. K and V tiles are stored row-major in LDS (XOR-swizzled,
//    double-buffered); the V^T operand comes straight from the gfx950
//    transposing LDS read (ds_read_b64_tr_b16), so V is never transposed in
//    registers. The next key block's global loads are in flight while the
//    current one is computed. Pad keys of partial blocks are masked from a
//    per-block 128-bit validity mask (computed once per call). Two instances:
//    <false> reads the block-ordered [H, Np, d] tensors; <true> reads the
//    token-order [H, N, d] tensors and does the block gather in its own tile
//    loads (per-block buffer resources based at the block's origin token),
//    so no block-ordered copy of Q, K or V is ever stored.
//  * attn_fwd_scalar: any dtype (fp32 / bf16), d in {64, 128}, B in {64, 128}.
//    One thread per query slot, fp32 online softmax, K/V staged through LDS as
//    fp32. This is the exact-parity path (fp32 inputs) and the fallback.
#include <mutex>

#include "attn_common.hpp"
#include "bsa.h"
#include "kernels.hpp"

namespace bsa {
namespace {

// ------------------------------------------------------------ scalar path --
template <typename T, int D>
__global__ __launch_bounds__(128) void attn_fwd_scalar(Lay L, const int32_t* zone_shape,
                                                       const T* qp, const T* kp, const T* vp,
                                                       const int32_t* counts, const int32_t* idx,
                                                       float scale, T* op, float* lse) {
  extern __shared__ float smem[];
  float* ks = smem;               // [B][D]
  float* vs = smem + L.B * D;     // [B][D]
  const int i = blockIdx.x, h = blockIdx.y, r = threadIdx.x;
  const size_t row = (size_t)h * L.M + i;
  const int n = counts[row];
  const int32_t* lst = idx + row * L.M;
  const size_t qoff = ((size_t)h * L.Np + (size_t)i * L.B + r) * D;
  float q[D], o[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = to_f32(qp[qoff + e]) * scale;
    o[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int it = 0; it < n; ++it) {
    const int j = lst[it];
    const Box xj = block_box(L, zone_shape, j);
    __syncthreads();
    const size_t koff = ((size_t)h * L.Np + (size_t)j * L.B) * D;
    for (int e = r; e < L.B * D; e += blockDim.x) {
      ks[e] = to_f32(kp[koff + e]);
      vs[e] = to_f32(vp[koff + e]);
    }
    __syncthreads();
    for (int c = 0; c < L.B; ++c) {
      if (!slot_real(xj, c)) continue;
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) s = fmaf(q[e], ks[c * D + e], s);
      if (s > m) {
        const float corr = expf(m - s);
        l *= corr;
#pragma unroll
        for (int e = 0; e < D; ++e) o[e] *= corr;
        m = s;
      }
      const float p = expf(s - m);
      l += p;
#pragma unroll
      for (int e = 0; e < D; ++e) o[e] = fmaf(p, vs[c * D + e], o[e]);
    }
  }
  const float inv = n > 0 ? 1.f / l : 0.f;
#pragma unroll
  for (int e = 0; e < D; ++e) op[qoff + e] = from_f32<T>(o[e] * inv);
  lse[(size_t)h * L.Np + (size_t)i * L.B + r] = n > 0 ? m + logf(l) : -INFINITY;
}

// -------------------------------------------------------------- MFMA path --
constexpr int kD = 128;          // head dim
constexpr int kB = 128;          // tokens per block (queries and keys)
constexpr int kTile = kB * kD;   // bf16 elements of one K or V tile (32 KB)
constexpr int kThreads = 512;    // 8 wavefronts
constexpr float kLazy = 8.f;     // log2 headroom of the lazily updated softmax max
constexpr int kMaxList = BSA_MAX_BLOCKS;  // longest key-block list of a row

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// LDS tiles are row-major (row = token, 256 bytes = 16 chunks of 16 bytes) with
// an XOR swizzle of the chunk index: K chunk q of row r sits at q ^ (r & 15),
// V chunk q at q ^ 4 (r & 3). With these, the K operand reads (16 rows x one
// chunk per 16-lane phase) and the V transposed reads (4 rows x 64 bytes per
// 32-lane phase) are bank-conflict free.
__device__ inline int kswz(int r, int q) { return q ^ (r & 15); }
__device__ inline int vswz(int r, int q) { return q ^ ((r & 3) << 2); }

// Tiles arrive by direct global->LDS loads (16 bytes per lane): load m
// (0..3) of wave w fills LDS slots (8m + w) * 64 + lane, i.e. row
// 4 (8m + w) + lane / 16, physical chunk lane % 16; the lane therefore fetches
// the logical chunk that the swizzle puts there. `src` is the byte offset of
// the block inside the head's tensor (the buffer resource covers the head).
template <bool kIsV>
__device__ inline void dma_part(__bf16* tile, const i32x4& rsrc, int src, int w, int lane, int m) {
  const int r = 4 * (8 * m + w) + (lane >> 4);
  const int q = kIsV ? vswz(r, lane & 15) : kswz(r, lane & 15);
  dma16_manual(rsrc, lds_addr_of(tile + (8 * m + w) * 512), 2 * (r * kD + 8 * q), src);
}
template <bool kIsV>
__device__ inline void dma_tile(__bf16* tile, const i32x4& rsrc, int src, int w, int lane) {
#pragma unroll
  for (int m = 0; m < 4; ++m) dma_part<kIsV>(tile, rsrc, src, w, lane, m);
}

// Gathered tiles (rows read straight from the token-order [H, N, d] tensors).
// Every block shape here has a width that is a multiple of 4, so the four
// rows 4g .. 4g + 3 of a load are four consecutive raster tokens: the load's
// source is the row group's token, origin + rel(g), plus the lane's own part
// (row 4g + lane / 16, the chunk its swizzle asks for). rel(g) is the raster
// offset of slot 4g inside a block of shape s, times the 256-byte row. The
// buffer resource of a block starts at its origin's row and ends at the
// head's last token, so a load's offset is rel(g) plus the lane's part (the
// same for every block of one shape) and the hardware range check turns a pad
// row past the last token into zeros.
// (s uniform over the wavefront, so that L.sh[s] is a scalar load: indexed by
// a per-lane id it would be a vector load, waited for behind every load in
// flight)
__device__ inline int group_rel_bytes(const Lay& L, int s, int g) {
  const int bw = L.sh[s][2], bh = L.sh[s][1];
  const int r = 4 * g;
  const int rw = r % bw, rh = (r / bw) % bh, rt = r / (bw * bh);
  return 2 * kD * ((rt * L.H + rh) * L.W + rw);
}
// The lane's part: row lane / 16 of the group, its swizzled chunk. It does not
// depend on the group (the swizzles see row & 15 = (4 g + lane / 16) & 15 with
// g = 8m + w', and 4 g & 15 = 4 w' & 15, the same for w' = w and w + 4).
template <bool kIsV>
__device__ inline int gather_lane_off(int w, int lane) {
  const int u = lane >> 4, r = 4 * w + u;
  const int q = kIsV ? vswz(r, lane & 15) : kswz(r, lane & 15);
  return 2 * (u * kD + 8 * q);
}
// Part m (0..3) of wave w (0..7): LDS slots (8m + w) * 64 + lane, row group
// g = 8m + w, from byte `voff` (rel(g) plus the lane's part) of the block's
// resource.
__device__ inline void dma_gather(__bf16* tile, const i32x4& rsrc, int voff, int w, int m) {
  dma16_manual(rsrc, lds_addr_of(tile + (8 * m + w) * 512), voff, 0);
}
// The resource of a block whose origin is token `origin` of a head starting at
// `head`: rows origin .. N-1 (none for an origin past the last token).
__device__ inline i32x4 block_rsrc(const __bf16* head, long long n_tokens, int origin) {
  origin = __builtin_amdgcn_readfirstlane(origin);  // (uniform: the resource is scalar)
  const long long rows = n_tokens > origin ? n_tokens - origin : 0;
  return make_buffer_rsrc(head + (size_t)origin * kD,
                          (uint32_t)__builtin_amdgcn_readfirstlane((int)(rows * kD * 2)));
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8): vmcnt(0) and lgkmcnt(0), each leaving the others free. Issued
// as builtins so that the compiler's own wait-count tracking sees them.
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitLgkm0 = 0xC07F;

// Workgroup barrier without the memory fence of __syncthreads(): that fence
// would also wait for every tile load still in flight. Each wave waits for the
// loads the next phase needs before arriving here; the "memory" clobber keeps
// the compiler from moving LDS accesses across the barrier.
__device__ inline void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Keeps the compiler's scheduler from moving instructions across this point, so
// that a phase's LDS reads are all issued before its matrix instructions.
__device__ inline void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// max / sum of a value over the lane pair (l, l ^ 32)
__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline bf16x4 tr_read(const __bf16* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// The validity words of one key block for this wave's 64 keys.
struct HalfMeta {
  uint32_t w0, w1;  // bits of keys 64kh + 0..31 and 64kh + 32..63
  int count;        // real slots of the block (128 = full, no pad keys)
};

// The first four k-steps' K fragments of S^T (for qk_tiles_pre), requested
// by the caller during the products before it.
__device__ inline void k_frags(bf16x8 (&a)[4][2], const __bf16* sk, int koff, int kswz_lane, int hi,
                               int st0) {
#pragma unroll
  for (int st = st0; st < st0 + 2; ++st)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
      a[st][kt] = *reinterpret_cast<const bf16x8*>(sk + koff + 32 * kt * kD +
                                                   8 * ((2 * st + hi) ^ kswz_lane));
}
template <typename Hook>
__device__ inline void qk_tiles_pre(f32x16 (&s)[2], const __bf16* sk, int koff, int kswz_lane,
                                    const bf16x8 (&qf)[8], int l32, int hi, const HalfMeta& m,
                                    const bf16x8& bias_b, const bf16x8 (&pre)[4][2], Hook hook) {
  bf16x8 a[8][2];
  auto load = [&](int st) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
      a[st][kt] = *reinterpret_cast<const bf16x8*>(sk + koff + 32 * kt * kD +
                                                   8 * ((2 * st + hi) ^ kswz_lane));
  };
#pragma unroll
  for (int st = 0; st < 4; ++st)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) a[st][kt] = pre[st][kt];
  // k-step 0 starts from the pad-key bias (partial block) or from an
  // immediate zero accumulator (full block: no register clearing)
  const f32x16 zero = {};
  if (__builtin_amdgcn_readfirstlane(m.count) < kB) {
    s[0] = mfma32x32x16(pad_bias_a(m.w0, l32, hi), bias_b, zero);
    s[1] = mfma32x32x16(pad_bias_a(m.w1, l32, hi), bias_b, zero);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) s[kt] = mfma32x32x16(a[0][kt], qf[0], s[kt]);
  } else {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) s[kt] = mfma32x32x16(a[0][kt], qf[0], zero);
  }
  load(4);
  hook(0);
  sched_fence();
#pragma unroll
  for (int st = 1; st < 8; ++st) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) s[kt] = mfma32x32x16(a[st][kt], qf[st], s[kt]);
    if (st + 4 < 8) load(st + 4);
    hook(st);
    sched_fence();
  }
}

// S^T = K Q^T for this wave's 64 keys of the block in `sk` (two 32x32 tiles),
// starting from the pad-key bias when the block is partial. The K fragments
// are requested four k-steps (eight products) ahead of the products that
// consume them.
template <typename Hook>
__device__ inline void qk_tiles(f32x16 (&s)[2], const __bf16* sk, int koff, int kswz_lane,
                                const bf16x8 (&qf)[8], int l32, int hi, const HalfMeta& m,
                                const bf16x8& bias_b, Hook hook) {
  bf16x8 a[8][2];
  auto load = [&](int st) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
      a[st][kt] = *reinterpret_cast<const bf16x8*>(sk + koff + 32 * kt * kD +
                                                   8 * ((2 * st + hi) ^ kswz_lane));
  };
#pragma unroll
  for (int st = 0; st < 4; ++st) load(st);
  sched_fence();
  // k-step 0 starts from the pad-key bias (partial block) or from an
  // immediate zero accumulator (full block: no register clearing)
  const f32x16 zero = {};
  if (__builtin_amdgcn_readfirstlane(m.count) < kB) {
    s[0] = mfma32x32x16(pad_bias_a(m.w0, l32, hi), bias_b, zero);
    s[1] = mfma32x32x16(pad_bias_a(m.w1, l32, hi), bias_b, zero);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) s[kt] = mfma32x32x16(a[0][kt], qf[0], s[kt]);
  } else {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) s[kt] = mfma32x32x16(a[0][kt], qf[0], zero);
  }
  load(4);
  hook(0);
  sched_fence();
#pragma unroll
  for (int st = 1; st < 8; ++st) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) s[kt] = mfma32x32x16(a[st][kt], qf[st], s[kt]);
    if (st + 4 < 8) load(st + 4);
    hook(st);
    sched_fence();
  }
}

// O^T (d x queries) += V^T (d x keys) P^T (keys x queries) over this wave's 64
// keys. P^T fragment c (c = 0..3) holds keys 16c + 8(jj/4) + 4hi + jj%4
// (jj = 0..7); the transposed V reads produce the same key order. The reads of
// two d-tiles are in flight ahead of the products that use them.
template <typename Hook>
__device__ inline void pv_tiles(f32x16 (&o)[4], const __bf16* sv, const int (&voff)[4],
                                const bf16x8 (&pf8)[4], Hook hook) {
  bf16x8 a[4][4];
  auto load = [&](int t) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const __bf16* p0 = sv + voff[t] + 16 * c * kD;
      const bf16x4 lo = tr_read(p0);
      const bf16x4 up = tr_read(p0 + 8 * kD);
      a[t][c] = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  load(0);
  load(1);
  sched_fence();
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (t + 2 < 4) load(t + 2);
#pragma unroll
    for (int c = 0; c < 4; ++c) o[t] = mfma32x32x16(a[t][c], pf8[c], o[t]);
    hook(t);
    sched_fence();
  }
}

// kGather: qp, kp, vp are the token-order [H, N, d] tensors (the block
// order is applied inside the tile loads) and the output is in raster order.
template <bool kGather>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_mfma(
    Lay L, const BlockMeta* __restrict__ meta, const __bf16* __restrict__ qp,
    const __bf16* __restrict__ kp, const __bf16* __restrict__ vp,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ idx, float scale_log2,
    __bf16* __restrict__ op, float* __restrict__ lse, const int32_t* __restrict__ zone_shape,
    int raster) {
  // (the swizzles assume 256-byte aligned tile rows)
  __shared__ __align__(1024) __bf16 sK[2][kTile];  // 2 x 32 KB
  __shared__ __align__(1024) __bf16 sV[2][kTile];  // 2 x 32 KB
  // The row's key-block list (16 KB): block ids, or gathered, each block's
  // origin and shape packed as origin * 4 + shape (the ids then sit in sB).
  __shared__ int32_t sL[kMaxList];
  __shared__ uint16_t sB[kGather ? kMaxList : 2];
  __shared__ __align__(16) uint32_t sM[2][64];   // block facts of blocks j, j+1 (8 copies each)
  __shared__ __align__(16) int sRel[kGather ? 4 * 32 : 4];  // rel(g) bytes, [shape][w][k]
  int i, h;  // (query block, head)
  xcd_item(i, h);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qg = w & 3, kh = w >> 2;
  const int l32 = lane & 31, hi = lane >> 5;
  const size_t row = (size_t)h * L.M + i;
  const int32_t* lst = idx + row * L.M;
  const size_t head0 = (size_t)h * L.Np;
  const int q = 32 * qg + l32;  // this lane's query inside the block
  // One memory round trip for the row's count, its list (every row has room
  // for M entries; they are read ahead of the count and kept only where the
  // count covers them) and this lane's Q^T fragments (B operand of S^T = K Q^T:
  // Q[q][16s + 8hi .. +8]).
  const int n = __builtin_amdgcn_readfirstlane(counts[row]);
  const int blk0_list = __builtin_amdgcn_readfirstlane(lst[0]);
  const int blk1_list = __builtin_amdgcn_readfirstlane(L.M > 1 ? lst[1] : 0);
  constexpr int kLU = kMaxList / kThreads;  // list entries per thread
  int ent[kLU];
#pragma unroll
  for (int u = 0; u < kLU; ++u) {
    const int e = tid + u * kThreads;
    ent[u] = e < L.M ? lst[e] : 0;
  }
  // where this lane's output row goes: its slot of the permuted [H, Np, d]
  // layout, or (raster) its token's row of [H, N, d] (pad slots: nowhere);
  // gathered, the query row comes from that token's row too (a pad slot reads
  // token 0 and writes nothing)
  size_t orow_i = head0 + (size_t)i * kB + q;
  bool o_real = true;
  bf16x8 qf[8];
  if (!kGather) {
    const __bf16* qrow = qp + (head0 + (size_t)i * kB + q) * kD + 8 * hi;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s);
  }
  if (kGather) {
    // from the query block's table entry (no zone-shape lookup): slot q is
    // real iff its mask bit is set, and then its token is the block's origin
    // plus the slot's raster offset in the block's shape
    const BlockMeta& mi = meta[i];
    const int si = __builtin_amdgcn_readfirstlane(mi.shape());
    const int bw = L.sh[si][2], bh = L.sh[si][1];
    const int k = q >> 5;
    const uint32_t word = k == 0 ? mi.half[0][0] : k == 1 ? mi.half[0][1]
                          : k == 2 ? mi.half[1][0] : mi.half[1][1];
    o_real = (word >> (q & 31)) & 1u;
    const int rel = ((q / (bw * bh)) * L.H + (q / bw) % bh) * L.W + q % bw;
    orow_i = (size_t)h * L.N + (size_t)(o_real ? (long long)mi.origin() + rel : 0);
  } else if (raster) {
    const long long tok = slot_token(L, block_box(L, zone_shape, i), q);
    o_real = tok >= 0;
    orow_i = (size_t)h * L.N + (size_t)(o_real ? tok : 0);
  }
  if (kGather) {  // a pad slot's query is zero, as in the permuted layout
    const __bf16* qrow = qp + orow_i * kD + 8 * hi;
    const bf16x8 zq = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(qrow + 16 * s);
      qf[s] = o_real ? x : zq;
    }
  }

  if (n == 0) {  // empty list (an all-pad query block): zeros, lse = -inf
    if (kh == 0 && o_real) {
      __bf16* orow = op + orow_i * kD;
      for (int e = 8 * hi; e < kD; e += 16) *reinterpret_cast<uint4*>(orow + e) = make_uint4(0, 0, 0, 0);
      if (hi == 0) lse[orow_i] = -INFINITY;
    }
    return;
  }
  // the buffer resources cover the head's rows: Np permuted slots, or N
  // tokens (gathered: a pad row's source past the last token reads zeros)
  const size_t src0 = kGather ? (size_t)h * L.N : head0;
  const uint32_t head_bytes = (uint32_t)((kGather ? (size_t)L.N : (size_t)L.Np) * kD * 2);
  const i32x4 krs = make_buffer_rsrc(kp + src0 * kD, head_bytes);
  const i32x4 vrs = make_buffer_rsrc(vp + src0 * kD, head_bytes);
  const i32x4 mrs = make_buffer_rsrc(meta, (uint32_t)L.M * sizeof(BlockMeta));
  constexpr int kTileBytes = kTile * 2;

  // Block facts travel like the tiles: wave 0 copies block blk's 32-byte
  // record into slot sM[slot] (each lane one dword; eight copies), and every
  // wave reads its half (validity words of its 64 keys, real-slot count) from
  // there after the barrier that follows the wait.
  auto fetch_meta = [&](int blk, int slot) {
    if (w == 0) dma4_manual(mrs, lds_addr_of(&sM[slot][0]), 4 * (lane & 7), blk * 32);
  };
  auto read_meta = [&](int slot) {
    typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
    const u32x3 v = *reinterpret_cast<const u32x3*>(&sM[slot][4 * kh]);
    return HalfMeta{v.x, v.y, (int)v.z};
  };
  auto uniform = [](const HalfMeta& m) {
    return HalfMeta{(uint32_t)__builtin_amdgcn_readfirstlane(m.w0),
                    (uint32_t)__builtin_amdgcn_readfirstlane(m.w1),
                    __builtin_amdgcn_readfirstlane(m.count)};
  };

  // prologue: tiles K0, V0 (and K1), block 0's mask words; then the list
  // into LDS (after the tile loads are on their way)
  const int blk0 = blk0_list;
  const int blk1 = n > 1 ? blk1_list : 0;
  // gathered loads: this lane's parts of the K and V row groups, and the
  // rel(g) table of every shape for the loop's loads (waves 0..3, loads k)
  const __bf16* k_head = kp + src0 * kD;
  const __bf16* v_head = vp + src0 * kD;
  const int lane_k = kGather ? gather_lane_off<false>(w, lane) : 0;
  const int lane_v = kGather ? gather_lane_off<true>(w, lane) : 0;
  if (kGather) {
    for (int s = 0; s < L.n_shapes; ++s)
      if (tid < 32) sRel[32 * s + tid] = group_rel_bytes(L, s, ((tid >> 3) & 3) + 4 * (tid & 7));
    const int s0 = __builtin_amdgcn_readfirstlane(meta[blk0].shape());
    const int s1 = __builtin_amdgcn_readfirstlane(meta[blk1].shape());
    const int o0 = __builtin_amdgcn_readfirstlane((int)meta[blk0].origin());
    const int o1 = __builtin_amdgcn_readfirstlane((int)meta[blk1].origin());
    const i32x4 k0 = block_rsrc(k_head, L.N, o0), v0 = block_rsrc(v_head, L.N, o0);
    const i32x4 k1 = block_rsrc(k_head, L.N, o1);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int r0 = group_rel_bytes(L, s0, 8 * m + w);
      dma_gather(sK[0], k0, lane_k + r0, w, m);
      dma_gather(sV[0], v0, lane_v + r0, w, m);
      dma_gather(sK[1], k1, lane_k + group_rel_bytes(L, s1, 8 * m + w), w, m);
    }
  } else {
    dma_tile<false>(sK[0], krs, blk0 * kTileBytes, w, lane);
    dma_tile<true>(sV[0], vrs, blk0 * kTileBytes, w, lane);
    dma_tile<false>(sK[1], krs, blk1 * kTileBytes, w, lane);  // (block 0 again if n = 1)
  }
  fetch_meta(blk0, 0);
  fetch_meta(blk1, 1);
#pragma unroll
  for (int u = 0; u < kLU; ++u) {
    const int e = tid + u * kThreads;
    if (e < n) {
      if (kGather) {
        sB[e] = (uint16_t)ent[u];
        sL[e] = (int)meta[ent[u]].origin() * 4 + meta[ent[u]].shape();
      } else {
        sL[e] = ent[u];
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

  // K operand (A of S^T): row 64kh + 32kt + l32, chunk (2st + hi) ^ (l32 & 15).
  const int koff = (64 * kh + l32) * kD;
  const int kswz_lane = l32 & 15;
  // V transposed read: lane (G = lane >> 4, u = lane & 15) supplies the 8 bytes
  // of row R + (u >> 2), columns 32t + 16(G & 1) + 4(u & 3) .. +4, and receives
  // V[R + 0..3][32t + l32] (R = 64kh + 16c + 4hi, second read R + 8).
  const int G = lane >> 4, u = lane & 15;
  const int vy = u >> 2, vx = 2 * (G & 1) + ((u & 3) >> 1);
  int voff[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    voff[t] = (64 * kh + 4 * hi + vy) * kD + 8 * (4 * (t ^ vy) + vx) + 4 * (u & 1);

  const bf16x8 bias_b = pad_bias_b(hi);
  f32x16 o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  float m_run = -INFINITY;  // reference max of s * scale * log2(e)
  float l_run = 0.f;        // this lane's share of the running sum
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
  f32x16 s_cur[2];

  // nothing from the scalar path may be outstanding inside the loop: there
  // the LDS reads are waited for by count, in issue order
  asm volatile("" ::"s"(scale_log2));
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __syncthreads();
  HalfMeta meta_j = uniform(read_meta(0));

  auto softmax = [&](bf16x8 (&pf8)[4], auto hook) {
    // Online softmax (log2 domain) with a lazily updated reference max: the
    // exponent base m_run moves only when a row max exceeds it by more than
    // kLazy (then p <= 2^kLazy, safe in bf16 and fp32), so O is rarely
    // rescaled.
    float mxa = fmaxf(s_cur[0][0], s_cur[0][1]), mxb = fmaxf(s_cur[1][0], s_cur[1][1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) {
      mxa = fmaxf(mxa, s_cur[0][r]);
      mxb = fmaxf(mxb, s_cur[1][r]);
    }
    const float mx = pair_max(fmaxf(mxa, mxb)) * scale_log2;
    if (__ballot(mx > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2_fast(m_run - (m_new == -INFINITY ? 0.f : m_new));
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pf8[2 * kt + (r >> 3)][r & 7] = (__bf16)exp2_fast(fmaf(s_cur[kt][r], scale_log2, -m_use));
        if (r & 1) {  // a fixed spot in the instruction stream for the caller's loads
          sched_fence();
          hook(8 * kt + (r >> 1));
          sched_fence();
        }
      }
  };
  // Row sum of the rounded probabilities (the weights the products use),
  // taken after PV in the matrix half: it reads the same P registers, and its
  // vector instructions then sit between matrix instructions instead of
  // lengthening the exponential half.
  auto rowsum = [&](const bf16x8 (&pf8)[4]) {
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      ps[c] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf8[c], pf8[c], 0, 1), ones,
                                              ps[c], false);
      ps[c] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf8[c], pf8[c], 2, 3), ones,
                                              ps[c], false);
      ps[c] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf8[c], pf8[c], 4, 5), ones,
                                              ps[c], false);
      ps[c] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf8[c], pf8[c], 6, 7), ones,
                                              ps[c], false);
    }
    l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
  };
  auto no_hook = [](int) {};

  // Ping-pong schedule. Each SIMD runs one wave of each key half (kh = 0, 1).
  // Iteration j has a matrix half (PV_j, then S_{j+1}) and an exponential half
  // (the softmax of one block); the two waves run them in opposite orders, so
  // that while one wave exponentiates, the other keeps the SIMD's matrix unit
  // busy:
  //   kh = 0:  softmax_j           , PV_j, S_{j+1}
  //   kh = 1:  PV_j, S_{j+1}       , softmax_{j+1}
  // No barrier separates the halves (nothing is handed between the waves
  // there; each wave runs its own order and the SIMD interleaves them, which
  // measured 3-4% faster than holding both to the halves). Iteration j reads
  // K_{j+1} and V_j, and requests K_{j+2} and V_{j+1} (into the buffers that
  // K_j and V_{j-1} left in iteration j-1) and the facts of block j+2; all of
  // them are waited for at its end, before its one barrier. Only the kh = 0
  // waves issue these loads, one every two exponentials: the global-to-LDS
  // path drains about 64 bytes per clock per CU, a wave that issues into a
  // full queue stalls, and the exponentiating wave has slack where the matrix
  // wave has none. The loads carry no branch (a branch between the
  // exponentials lets the compiler sink the exponentials past all sixteen
  // loads, which then leave as one burst and stall the wave for about a
  // thousand cycles). In the matrix half, the last two d-tiles of PV_j request
  // the first four k-steps of K fragments of S_{j+1}, so the S products start
  // without waiting on LDS.
  // Buffer ownership: iteration 0 refills sK[0] (with K_2) and sM[0] (with the
  // facts of block 2), which every wave reads before the loop (S_0 and block 0's
  // facts); the barrier after S_0 keeps those refills behind the last of
  // these reads. From then on, a buffer is refilled only in the iteration after
  // the one that read it, past that iteration's closing barrier.
  auto walk = [&](auto khc) {
    constexpr int KH = decltype(khc)::value;
    // Pad halves. When a block's upper 64 keys are all pad (the last frames
    // of a block that sticks out of a grid of 13 frames, say), the kh = 1
    // wave's scores there all carry the pad bias and add nothing to O or the
    // row sum. That wave then skips S and the exponentials of the block and
    // sets its P to zero. It still runs the block's PV product (exact zeros
    // added) when the next block has real keys, and skips it only when the
    // next block is a pad half too or there is none: so its matrix half keeps
    // facing the other wave's exponentials. Skipping the PV product as well
    // made the wave's next exponentials overlap the other wave's, and the
    // kernel slower. The decision is per block and half, the same in every
    // lane; S and the exponentials of block 0 are always computed (before the
    // loop).
    bool skip_cur = KH == 1 && (meta_j.w0 | meta_j.w1) == 0u;
    qk_tiles(s_cur, sK[0], koff, kswz_lane, qf, l32, hi, meta_j, bias_b, no_hook);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    barrier();
    bf16x8 pf8[4];
    if (KH == 1) softmax(pf8, no_hook);
    // list entries of blocks j+1 and j+2 (ids, or gathered, packed origins and
    // shapes; then also block j+2's id), carried in scalar registers; the next
    // ones are read from LDS an iteration ahead
    int b1 = __builtin_amdgcn_readfirstlane(sL[min(1, n - 1)]);
    int b2 = __builtin_amdgcn_readfirstlane(sL[min(2, n - 1)]);
    int id2 = kGather ? __builtin_amdgcn_readfirstlane((int)sB[min(2, n - 1)]) : 0;
    // gathered: the offsets of this wave's eight K and eight V loads for the
    // shape they were last formed for (re-formed when a block's shape differs)
    int vk[8] = {}, vv[8] = {};
    int sk_cur = -1, sv_cur = -1;
    for (int j = 0; j < n; ++j) {
      const int cb = j & 1, nb = cb ^ 1;
      const bool more1 = j + 1 < n, more2 = j + 2 < n;
      const int b3 = sL[min(j + 3, n - 1)];
      const int id3 = kGather ? (int)sB[min(j + 3, n - 1)] : 0;
      typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
      const u32x3 mraw = *reinterpret_cast<const u32x3*>(&sM[nb][4 * kh]);
      // gathered: the resources of K_{j+2} (block j+2's origin) and V_{j+1}
      // (block j+1's), and the load offsets of their shapes
      i32x4 krs_t = krs, vrs_t = vrs;
      if (kGather && KH == 0) {
        const int sk = b2 & 3, sv = b1 & 3;
        krs_t = block_rsrc(k_head, L.N, b2 >> 2);
        vrs_t = block_rsrc(v_head, L.N, b1 >> 2);
        if (sk != sk_cur) {
#pragma unroll
          for (int k = 0; k < 8; ++k) vk[k] = lane_k + sRel[32 * sk + 8 * w + k];
          sk_cur = sk;
        }
        if (sv != sv_cur) {
#pragma unroll
          for (int k = 0; k < 8; ++k) vv[k] = lane_v + sRel[32 * sv + 8 * w + k];
          sv_cur = sv;
        }
      }
      // wave w (kh = 0) fills parts (w, m) and (w + 4, m) of K_{j+2} and V_{j+1}
      // Issued unconditionally (no branch between the exponentials, so the
      // loads stay spread over them): past the end of the list b1 and b2 repeat
      // the last block, and the buffers they fill are free and never read again.
      auto dma_hook = [&](int k) {
        const int ww = w + 4 * (k & 1), m = (k >> 1) & 3;
        if (kGather) {
          if (k < 8)
            dma_gather(sK[cb], krs_t, vk[k], ww, m);
          else
            dma_gather(sV[nb], vrs_t, vv[k - 8], ww, m);
        } else {
          if (k < 8)
            dma_part<false>(sK[cb], krs, b2 * kTileBytes, ww, lane, m);
          else
            dma_part<true>(sV[nb], vrs, b1 * kTileBytes, ww, lane, m);
        }
      };
      if (KH == 0 && more2) fetch_meta(kGather ? id2 : b2, cb);
      const HalfMeta meta_n{mraw.x, mraw.y, (int)mraw.z};
      if (KH == 0) {
        softmax(pf8, dma_hook);
        bf16x8 kpre[4][2];
        auto kpre_hook = [&](int t) {
          if (t >= 2) k_frags(kpre, sK[nb], koff, kswz_lane, hi, 2 * (t - 2));
        };
        pv_tiles(o, sV[cb], voff, pf8, kpre_hook);
        rowsum(pf8);
        if (more1) {
          qk_tiles_pre(s_cur, sK[nb], koff, kswz_lane, qf, l32, hi, meta_n, bias_b, kpre, no_hook);
        }
      } else {
        const bool skip_n = __builtin_amdgcn_readfirstlane(mraw.x | mraw.y) == 0;
        bf16x8 kpre[4][2];
        auto kpre_hook = [&](int t) {
          if (t >= 2) k_frags(kpre, sK[nb], koff, kswz_lane, hi, 2 * (t - 2));
        };
        if (!(skip_cur && (skip_n || !more1))) {
          pv_tiles(o, sV[cb], voff, pf8, kpre_hook);
          rowsum(pf8);
        }
        if (more1 && !skip_n) {
          qk_tiles_pre(s_cur, sK[nb], koff, kswz_lane, qf, l32, hi, meta_n, bias_b, kpre, no_hook);
          softmax(pf8, no_hook);
        } else {
          const bf16x8 z = {};
#pragma unroll
          for (int c = 0; c < 4; ++c) pf8[c] = z;
        }
        skip_cur = skip_n;
      }
      b1 = b2;
      b2 = __builtin_amdgcn_readfirstlane(b3);
      if (kGather) id2 = __builtin_amdgcn_readfirstlane(id3);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      barrier();
    }
  };
  if (kh == 0)
    walk(std::integral_constant<int, 0>());
  else
    walk(std::integral_constant<int, 1>());
  // the last iteration's (unused) K requests must land before LDS is reused
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();

  // merge the two key halves (waves w and w+4 share their 32 queries)
  l_run = pair_sum(l_run);
  // element e of lane (qg, lane) at xo[256 e] (64 KB), so that the 64 lanes of
  // each access hit 64 consecutive words (no bank conflicts)
  float* xo = reinterpret_cast<float*>(&sK[0][0]) + qg * 64 + lane;
  float* xm = reinterpret_cast<float*>(&sV[0][0]) + qg * 64 + lane;
  if (kh == 1) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[256 * (16 * t + r)] = o[t][r];
    xm[0] = m_run;
    xm[256] = l_run;
  }
  __syncthreads();
  if (kh == 0 && o_real) {
    const float m2 = xm[0], l2 = xm[256];
    const float mt = fmaxf(m_run, m2);
    const float mu = mt == -INFINITY ? 0.f : mt;
    const float a1 = exp2_fast(m_run - mu), a2 = exp2_fast(m2 - mu);
    const float lt = l_run * a1 + l2 * a2;
    const float inv = 1.f / lt;
    __bf16* orow = op + orow_i * kD;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int r = 4 * g + rr;
          v[rr] = (__bf16)((o[t][r] * a1 + xo[256 * (16 * t + r)] * a2) * inv);
        }
        *reinterpret_cast<bf16x4*>(orow + 32 * t + 8 * g + 4 * hi) = v;
      }
    if (hi == 0) lse[orow_i] = (mt + log2f(lt)) * kLn2;
  }
}

template <typename T>
hipError_t launch_scalar(const Lay& L, const int32_t* zone_shape, const void* qp, const void* kp,
                         const void* vp, const int32_t* counts, const int32_t* idx, int heads,
                         int d, float scale, void* op, float* lse, hipStream_t st) {
  dim3 grid(L.M, heads);
  const size_t shmem = 2 * (size_t)L.B * d * sizeof(float);
  const T* q = static_cast<const T*>(qp);
  const T* k = static_cast<const T*>(kp);
  const T* v = static_cast<const T*>(vp);
  T* o = static_cast<T*>(op);
  if (d == 64) {
    auto kern = attn_fwd_scalar<T, 64>;
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)shmem);
    if (e != hipSuccess) return e;
    kern<<<grid, L.B, shmem, st>>>(L, zone_shape, q, k, v, counts, idx, scale, o, lse);
  } else {
    auto kern = attn_fwd_scalar<T, 128>;
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)shmem);
    if (e != hipSuccess) return e;
    kern<<<grid, L.B, shmem, st>>>(L, zone_shape, q, k, v, counts, idx, scale, o, lse);
  }
  return hipGetLastError();
}

// Scratch memory of the allocation-free forward: the per-block table for the
// largest layout the library takes (BSA_MAX_BLOCKS blocks of 32 bytes,
// 128 KiB). Each GPU the library runs on holds its own copy until the process
// ends. In host code `scratch` names a host-side stand-in, not the device
// array: its device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = (size_t)BSA_MAX_BLOCKS * sizeof(BlockMeta);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

}  // namespace

hipError_t attn_fwd_static_scratch(void** ptr, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex lock;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(lock);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = kScratchBytes;
  return hipSuccess;
}

bool attn_fwd_uses_mfma(const Lay& L, int d, bool bf16) { return bf16 && d == kD && L.B == kB; }

size_t attn_fwd_workspace(const Lay& L, int d, bool bf16) {
  return attn_fwd_uses_mfma(L, d, bf16) ? (size_t)L.M * sizeof(BlockMeta) : 0;
}

bool attn_fwd_gather_ok(const Lay& L, int d, bool bf16) {
  if (!attn_fwd_uses_mfma(L, d, bf16)) return false;
  for (int s = 0; s < L.n_shapes; ++s)
    if (L.sh[s][2] % 4 != 0) return false;
  // every source byte offset (origin + rel(g) + the lane's part, below the
  // padded grid's Np rows) must fit the 32-bit signed offsets used
  return (long long)L.Np * kD * 2 < (1ll << 31);
}

hipError_t launch_attn_fwd(const Lay& L, const int32_t* zone_shape, const void* qp,
                           const void* kp, const void* vp, const int32_t* counts,
                           const int32_t* idx, int heads, int d, bool bf16, float scale,
                           void* op, float* lse, void* ws, hipStream_t st, bool raster,
                           bool gather) {
  if (gather && !attn_fwd_gather_ok(L, d, bf16)) return hipErrorInvalidValue;
  if (attn_fwd_uses_mfma(L, d, bf16)) {
    BlockMeta* meta = static_cast<BlockMeta*>(ws);
    hipError_t e = launch_block_meta(L, zone_shape, meta, st);
    if (e != hipSuccess) return e;
    dim3 grid(L.M, heads);
    if (gather)
      attn_fwd_mfma<true><<<grid, kThreads, 0, st>>>(
          L, meta, static_cast<const __bf16*>(qp), static_cast<const __bf16*>(kp),
          static_cast<const __bf16*>(vp), counts, idx, scale * kLog2e,
          static_cast<__bf16*>(op), lse, zone_shape, 1);
    else
      attn_fwd_mfma<false><<<grid, kThreads, 0, st>>>(
          L, meta, static_cast<const __bf16*>(qp), static_cast<const __bf16*>(kp),
          static_cast<const __bf16*>(vp), counts, idx, scale * kLog2e,
          static_cast<__bf16*>(op), lse, zone_shape, raster ? 1 : 0);
    return hipGetLastError();
  }
  if (raster) return hipErrorInvalidValue;  // (the raster output needs the MFMA kernel)
  if (bf16)
    return launch_scalar<__bf16>(L, zone_shape, qp, kp, vp, counts, idx, heads, d, scale, op,
                                 lse, st);
  return launch_scalar<float>(L, zone_shape, qp, kp, vp, counts, idx, heads, d, scale, op, lse,
                              st);
}

}  // namespace bsa

// Audio-to-video cross-attention layer: projections, multi-head attention of
// the video tokens over the audio tokens, output projection; forward and
// backward.
//
// Prism page (trawling.dev/post/2299), section on block composition matched to
// regional information: the zone's block shape uses the feature norm of the
// audio-to-video cross-attention, the layer in which video tokens attend to
// the audio tokens. Reading implemented (the page gives no layer definition):
// H heads of d = 128 channels, weights in [out, in] layout, no biases,
//   Q = X Wq^T, K = A Wk^T, V = A Wv^T, O_h = softmax(Q_h K_h^T / sqrt(d)) V_h,
//   Y = O Wo^T,
// with Q, K, V, O, Y (and in the backward dO, dQ, dK, dV) stored as bf16, all
// products accumulated in fp32.
//
// Kernels:
//  gemm_nt_kernel    C[M,N] = sum_k A[m][k] B[n][k] on bf16 MFMA (both operands
//                    k-contiguous), 128 x 128 tiles, 64-deep k steps staged in
//                    LDS (XOR-swizzled 16-byte chunks, double-buffered), fp32
//                    accumulation, bf16 or fp32 output (optionally added to C).
//  transpose16_kernel bf16 [R, Cc] -> [Cc, ldo], columns R..ldo-1 zero (so
//                    transposed rows are whole 16-byte chunks): 8 x 8 blocks per
//                    lane transposed in registers, 16-byte loads and stores.
//  xattn_fwd_kernel  per (256 queries, head): K_h, V_h of every audio token in
//                    LDS; per wave 32 queries, S^T = K Q^T and O^T += V^T P^T on
//                    MFMA over 64-key chunks with an online softmax; writes O
//                    (bf16) and lse (natural log, fp32).
//  xattn_delta_kernel  D[h][n] = dO_h[n] . O_h[n] (fp32).
//  xattn_bwd_dq_kernel per (256 queries, head), K_h and V_h in LDS as in the
//                    forward: S^T = K Q^T and dP^T = V dO^T on MFMA, P = exp(S
//                    scale - lse), dS = P (dP - D), dQ^T = K^T dS^T (K^T through
//                    transposed LDS reads); writes dQ (bf16, scaled) and its
//                    transpose (the dWq product's operand).
//  xattn_bwd_dkdv_kernel per (query split, 128 keys, head): each wave keeps its
//                    32 keys of K and V in registers; Q, dO tiles of 128
//                    queries with their lse and D stream through LDS; S = Q K^T,
//                    dP = dO V^T, then dV += P^T dO and dK += dS^T Q (dO and Q
//                    through transposed LDS reads); writes fp32 partial sums per
//                    split, which xattn_reduce_kernel adds in a fixed order
//                    (deterministic) into bf16 dK (scaled) and dV.
#include <math.h>

#include <algorithm>

#include "attn_common.hpp"
#include "kernels.hpp"

namespace bsa {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ inline bf16x4 tr_read4(const __bf16* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// ------------------------------------------------------------------- GEMM --
constexpr int kGM = 128, kGN = 128, kGK = 64;  // block tile
constexpr int kGThreads = 256;                 // 4 waves, 2 x 2, 64 x 64 each

__device__ inline int gswz(int row, int chunk) { return chunk ^ (row & 7); }

// Split-K (kchunk > 0): workgroup z covers k in [z kchunk, (z + 1) kchunk) and
// writes its fp32 partial tile to C + z M ldc (kOutF32, no kAccum).
template <bool kOutF32, bool kAccum>
__global__ __launch_bounds__(kGThreads) void gemm_nt_kernel(const __bf16* __restrict__ A, int lda,
                                                          const __bf16* __restrict__ B, int ldb,
                                                          int M, int N, int K, void* C, int ldc,
                                                          int kchunk) {
  __shared__ __align__(16) __bf16 sA[2][kGM * kGK];
  __shared__ __align__(16) __bf16 sB[2][kGN * kGK];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int m0 = blockIdx.y * kGM, n0 = blockIdx.x * kGN;
  const int wm = w >> 1, wn = w & 1;
  // loader: chunk e = tid + 256 u (u = 0..3) of a tile: row e / 8, chunk e % 8
  u32x4 ra[4], rb[4];
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  int klim = K;  // loads past klim read zero (the end of this workgroup's k range)
  auto gload = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + kGThreads * u, r = e >> 3, ch = e & 7;
      const int k = k0 + 8 * ch;
      ra[u] = (m0 + r < M && k < klim)
                  ? *reinterpret_cast<const u32x4*>(A + (size_t)(m0 + r) * lda + k) : z4;
      rb[u] = (n0 + r < N && k < klim)
                  ? *reinterpret_cast<const u32x4*>(B + (size_t)(n0 + r) * ldb + k) : z4;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + kGThreads * u, r = e >> 3, ch = e & 7;
      *reinterpret_cast<u32x4*>(&sA[buf][r * kGK + 8 * gswz(r, ch)]) = ra[u];
      *reinterpret_cast<u32x4*>(&sB[buf][r * kGK + 8 * gswz(r, ch)]) = rb[u];
    }
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  const int kbeg = kchunk > 0 ? blockIdx.z * kchunk : 0;
  const int kend = kchunk > 0 ? min(K, kbeg + kchunk) : K;
  const int nk = kend > kbeg ? (kend - kbeg + kGK - 1) / kGK : 0;
  klim = kend;
  if (kchunk > 0) C = static_cast<float*>(C) + (size_t)blockIdx.z * M * ldc;
  gload(kbeg);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kbeg + (kt + 1) * kGK);
#pragma unroll
    for (int s = 0; s < kGK / 16; ++s) {
      bf16x8 af[2], bf[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int r = 64 * wm + 32 * a + l32;
        af[a] = *reinterpret_cast<const bf16x8*>(&sA[buf][r * kGK + 8 * gswz(r, 2 * s + hi)]);
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int r = 64 * wn + 32 * b + l32;
        bf[b] = *reinterpret_cast<const bf16x8*>(&sB[buf][r * kGK + 8 * gswz(r, 2 * s + hi)]);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = mfma32x32x16(af[a], bf[b], acc[a][b]);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }
  // lane holds C[64 wm + 32 a + 8 (r/4) + 4 hi + r%4][64 wn + 32 b + l32]
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int n = n0 + 64 * wn + 32 * b + l32;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + 64 * wm + 32 * a + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (m >= M) continue;
        if constexpr (kOutF32) {
          float* c = static_cast<float*>(C) + (size_t)m * ldc + n;
          *c = kAccum ? *c + acc[a][b][r] : acc[a][b][r];
        } else {
          static_cast<__bf16*>(C)[(size_t)m * ldc + n] = (__bf16)acc[a][b][r];
        }
      }
    }
}

// Large-shape variant: 256 x 256 block tile, 8 waves of 64 x 128 (2 x 4 MFMA
// tiles, 8 products per 6 fragment reads), operands copied global -> LDS by
// direct buffer loads (the XOR swizzle applied on the fetch side: LDS slot s of
// a tile holds row s / 8, logical chunk (s % 8) ^ (row % 8)); rows past M or N
// read zero through the buffer bounds. Needs K % 64 == 0 and each operand's
// rows below 2^31 bytes from the tile's first row. Without a k split the tiles
// are taken in the L2-aware order (the tiles of one 256-row panel of A run on
// one XCD).
constexpr int kBM = 256, kBN = 256;
constexpr int kBThreads = 512;

template <bool kOutF32, bool kAccum>
__global__ __launch_bounds__(kBThreads) void gemm_nt_big_kernel(
    const __bf16* __restrict__ A, int lda, const __bf16* __restrict__ B, int ldb, int M, int N,
    int K, void* C, int ldc, int kchunk) {
  __shared__ __align__(16) __bf16 sA[2][kBM * kGK];
  __shared__ __align__(16) __bf16 sB[2][kBN * kGK];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  int tx = blockIdx.x, ty = blockIdx.y;
  if (gridDim.z == 1) xcd_item(tx, ty);
  const int m0 = ty * kBM, n0 = tx * kBN;
  const int wm = w >> 1, wn = w & 1;  // rows 64 wm .., columns 128 wn ..
  const uint32_t abytes = (uint32_t)std::min<long long>((long long)(M - m0) * lda * 2, 0x7fffffffLL);
  const uint32_t bbytes = (uint32_t)std::min<long long>((long long)(N - n0) * ldb * 2, 0x7fffffffLL);
  const i32x4 ars = make_buffer_rsrc(A + (size_t)m0 * lda, abytes);
  const i32x4 brs = make_buffer_rsrc(B + (size_t)n0 * ldb, bbytes);
  // this lane's slots: unit u = w + 8 j (j = 0..3) of each tile, slot 64 u + lane
  int aoff[4], boff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int sl = 64 * (w + 8 * j) + lane, r = sl >> 3, ch = (sl & 7) ^ (r & 7);
    aoff[j] = (r * lda + 8 * ch) * 2;
    boff[j] = (r * ldb + 8 * ch) * 2;
  }
  const int kbeg = kchunk > 0 ? blockIdx.z * kchunk : 0;
  const int kend = kchunk > 0 ? min(K, kbeg + kchunk) : K;
  const int nk = kend > kbeg ? (kend - kbeg) / kGK : 0;
  if (kchunk > 0) C = static_cast<float*>(C) + (size_t)blockIdx.z * M * ldc;
  auto issue = [&](int kt, int buf) {
    const int kb = (kbeg + kt * kGK) * 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int u = w + 8 * j;
      dma16_manual(ars, lds_addr_of(&sA[buf][u * 64 * 8]), aoff[j], kb);
      dma16_manual(brs, lds_addr_of(&sB[buf][u * 64 * 8]), boff[j], kb);
    }
  };
  f32x16 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  if (nk > 0) issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) issue(kt + 1, buf ^ 1);
#pragma unroll
    for (int s = 0; s < kGK / 16; ++s) {
      bf16x8 af[2], bf[4];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int r = 64 * wm + 32 * a + l32;
        af[a] = *reinterpret_cast<const bf16x8*>(&sA[buf][r * kGK + 8 * gswz(r, 2 * s + hi)]);
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int r = 128 * wn + 32 * b + l32;
        bf[b] = *reinterpret_cast<const bf16x8*>(&sB[buf][r * kGK + 8 * gswz(r, 2 * s + hi)]);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = mfma32x32x16(af[a], bf[b], acc[a][b]);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next stage has landed
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int n = n0 + 128 * wn + 32 * b + l32;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + 64 * wm + 32 * a + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (m >= M) continue;
        if constexpr (kOutF32) {
          float* c = static_cast<float*>(C) + (size_t)m * ldc + n;
          *c = kAccum ? *c + acc[a][b][r] : acc[a][b][r];
        } else {
          static_cast<__bf16*>(C)[(size_t)m * ldc + n] = (__bf16)acc[a][b][r];
        }
      }
    }
}

// -------------------------------------------------------------- transpose --
// bf16 [R, Cc] -> [Cc, ldo] for 16-byte aligned rows (lds, ldo, Cc multiples of 8). Lane
// (cb = lane % 8, rb = lane / 8) of wave w loads an 8 x 8 block, src rows r + 0..7 (one
// 16-byte load each; rows past R read as zeros) and columns c + 0..7, and stores its
// transpose as dst rows c + 0..7, columns r + 0..7 (one 16-byte store each). Every load and
// store instruction of a wave covers eight whole 128-byte row segments.
__global__ __launch_bounds__(256) void transpose16_kernel(const __bf16* __restrict__ src, int R,
                                                          int Cc, int lds,
                                                          __bf16* __restrict__ dst, int ldo) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + 8 * (lane & 7);
  const long long r = ((long long)blockIdx.y * 4 + w) * 64 + 8 * (lane >> 3);
  if (c >= Cc || r >= ldo) return;
  u32x4 in[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    in[i] = r + i < R ? *reinterpret_cast<const u32x4*>(src + (size_t)(r + i) * lds + c) : z;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    // dst row c + j, columns r + 2m and r + 2m + 1: element j of src rows r + 2m, r + 2m + 1
    u32x4 out;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t a = in[2 * m][j >> 1], b = in[2 * m + 1][j >> 1];
      out[m] = (j & 1) ? (a >> 16) | (b & 0xffff0000u) : (a & 0xffffu) | (b << 16);
    }
    *reinterpret_cast<u32x4*>(dst + (size_t)(c + j) * ldo + r) = out;
  }
}

// ------------------------------------------------- cross-attention forward --
constexpr int kXD = 128;          // head dim
constexpr int kXLd = kXD + 16;    // LDS row stride (elements): 288 bytes
constexpr int kXWaves = 8;        // 32 queries each
constexpr int kXQ = 32 * kXWaves; // queries per workgroup
constexpr int kXMaxNa = 256;      // audio tokens held in LDS

__global__ __launch_bounds__(64 * kXWaves) void xattn_fwd_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    int N, int Na, int na_pad, int D, float scale_log2, __bf16* __restrict__ o,
    float* __restrict__ lse) {
  __shared__ __align__(16) __bf16 sK[kXMaxNa * kXLd];  // [na_pad][kXLd]
  __shared__ __align__(16) __bf16 sV[kXMaxNa * kXLd];
  const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  // stage K_h and V_h (rows past Na zero)
  for (int e = tid; e < na_pad * 16; e += 64 * kXWaves) {
    const int r = e >> 4, ch = e & 15;
    u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
    if (r < Na) {
      kv = *reinterpret_cast<const u32x4*>(k + (size_t)r * D + h * kXD + 8 * ch);
      vv = *reinterpret_cast<const u32x4*>(v + (size_t)r * D + h * kXD + 8 * ch);
    }
    *reinterpret_cast<u32x4*>(sK + r * kXLd + 8 * ch) = kv;
    *reinterpret_cast<u32x4*>(sV + r * kXLd + 8 * ch) = vv;
  }
  // Q^T fragments: lane holds Q[n][16 s + 8 hi .. +8] (rows past N read row N-1)
  const long long n = (long long)blockIdx.x * kXQ + 32 * w + l32;
  const bool n_ok = n < N;
  const __bf16* qrow = q + (size_t)(n_ok ? n : N - 1) * D + h * kXD + 8 * hi;
  bf16x8 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s);
  __syncthreads();

  f32x16 oacc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  // V^T transposed reads: lane (G = lane / 16, u = lane % 16) addresses row
  // R + u / 4, columns 32 t + 16 (G % 2) + 4 (u % 4) .. +4 and receives
  // V[R + 0..3][32 t + l32]
  const int G = lane >> 4, u = lane & 15;
  const int vrow = u >> 2, vcol = 16 * (G & 1) + 4 * (u & 3);
  for (int c0 = 0; c0 < na_pad; c0 += 64) {
    f32x16 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[t][r] = 0.f;
      const __bf16* kr = sK + (c0 + 32 * t + l32) * kXLd + 8 * hi;
#pragma unroll
      for (int st = 0; st < 8; ++st)
        s[t] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(kr + 16 * st), qf[st], s[t]);
    }
    // lane holds key c0 + 32 t + 8 (r/4) + 4 hi + r%4 of query n; log2 units
    float cmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = c0 + 32 * t + 8 * (r >> 2) + 4 * hi + (r & 3);
        s[t][r] = key < Na ? s[t][r] * scale_log2 : -INFINITY;
        cmax = fmaxf(cmax, s[t][r]);
      }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);  // finite: every chunk holds a real key
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
    bf16x8 pf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int t = j >> 1, r = 4 * (2 * (j & 1) + (jj >> 2)) + (jj & 3);
        const float p = exp2f(s[t][r] - m_new);
        const __bf16 pb = (__bf16)p;
        pf[j][jj] = pb;
        psum += (float)pb;
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;
    // O^T[d][n] += sum over the chunk's keys V[key][d] P[n][key]; k-step j's
    // slot jj is key c0 + 32 (j/2) + 16 (j%2) + 8 (jj/4) + 4 hi + jj%4
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int R = c0 + 32 * (j >> 1) + 16 * (j & 1) + 4 * hi;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const __bf16* p0 = sV + (R + vrow) * kXLd + 32 * t + vcol;
        const bf16x4 lo = tr_read4(p0);
        const bf16x4 up = tr_read4(p0 + 8 * kXLd);
        const bf16x8 a = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[t] = mfma32x32x16(a, pf[j], oacc[t]);
      }
    }
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!n_ok) return;
  const float inv = 1.f / l_tot;
  // lane holds O[n][h d + 32 t + 8 g + 4 hi + 0..3] in oacc[t][4 g .. 4 g + 3]
  __bf16* orow = o + (size_t)n * D + h * kXD + 4 * hi;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 v4;
#pragma unroll
      for (int i = 0; i < 4; ++i) v4[i] = (__bf16)(oacc[t][4 * g + i] * inv);
      *reinterpret_cast<bf16x4*>(orow + 32 * t + 8 * g) = v4;
    }
  if (hi == 0) lse[(size_t)h * N + n] = (m_run + log2f(l_tot)) * kLn2;
}

// ------------------------------------------------ cross-attention backward --
__global__ __launch_bounds__(256) void xattn_delta_kernel(const __bf16* __restrict__ dO,
                                                          const __bf16* __restrict__ o, int N,
                                                          int heads, float* __restrict__ delta) {
  // 16 lanes per (token, head) row of 128 channels, 8 channels (16 bytes) each
  const long long item = ((long long)blockIdx.x * 256 + threadIdx.x) >> 4;  // (n, h) row
  const int c = threadIdx.x & 15;
  const bool ok = item < (long long)N * heads;
  const long long it = ok ? item : 0;
  const size_t base = (size_t)it * kXD + 8 * c;  // rows of D = heads * 128 are contiguous
  const bf16x8 a = *reinterpret_cast<const bf16x8*>(dO + base);
  const bf16x8 b = *reinterpret_cast<const bf16x8*>(o + base);
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc += (float)a[i] * (float)b[i];
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (ok && c == 0) {
    const long long n = it / heads;
    const int h = (int)(it - n * heads);
    delta[(size_t)h * N + n] = acc;
  }
}

__global__ __launch_bounds__(64 * kXWaves) void xattn_bwd_dq_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dO, const float* __restrict__ lse,
    const float* __restrict__ delta, int N, int Na, int na_pad, int D, float scale,
    __bf16* __restrict__ dq, __bf16* __restrict__ dqT, int npad) {
  __shared__ __align__(16) __bf16 sK[kXMaxNa * kXLd];
  __shared__ __align__(16) __bf16 sV[kXMaxNa * kXLd];
  const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  for (int e = tid; e < na_pad * 16; e += 64 * kXWaves) {
    const int r = e >> 4, ch = e & 15;
    u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
    if (r < Na) {
      kv = *reinterpret_cast<const u32x4*>(k + (size_t)r * D + h * kXD + 8 * ch);
      vv = *reinterpret_cast<const u32x4*>(v + (size_t)r * D + h * kXD + 8 * ch);
    }
    *reinterpret_cast<u32x4*>(sK + r * kXLd + 8 * ch) = kv;
    *reinterpret_cast<u32x4*>(sV + r * kXLd + 8 * ch) = vv;
  }
  const long long n = (long long)blockIdx.x * kXQ + 32 * w + l32;
  const bool n_ok = n < N;
  const long long nr = n_ok ? n : N - 1;
  const __bf16* qrow = q + (size_t)nr * D + h * kXD + 8 * hi;
  const __bf16* drow = dO + (size_t)nr * D + h * kXD + 8 * hi;
  bf16x8 qf[8], df[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    qf[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s);
    df[s] = *reinterpret_cast<const bf16x8*>(drow + 16 * s);
  }
  const float l2 = lse[(size_t)h * N + nr] * kLog2e;  // lse in log2 units
  const float dn = delta[(size_t)h * N + nr];
  const float sl2 = scale * kLog2e;
  __syncthreads();
  f32x16 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  const int G = lane >> 4, u = lane & 15;
  const int vrow = u >> 2, vcol = 16 * (G & 1) + 4 * (u & 3);
  for (int c0 = 0; c0 < na_pad; c0 += 64) {
    f32x16 s[2], dp[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[t][r] = dp[t][r] = 0.f;
      const __bf16* kr = sK + (c0 + 32 * t + l32) * kXLd + 8 * hi;
      const __bf16* vr = sV + (c0 + 32 * t + l32) * kXLd + 8 * hi;
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        s[t] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(kr + 16 * st), qf[st], s[t]);
        dp[t] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(vr + 16 * st), df[st], dp[t]);
      }
    }
    // dS (bf16) in the key order the dQ product takes: k-step j, slot jj =
    // key c0 + 32 (j/2) + 16 (j%2) + 8 (jj/4) + 4 hi + jj%4
    bf16x8 dsf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int t = j >> 1, r = 4 * (2 * (j & 1) + (jj >> 2)) + (jj & 3);
        const int key = c0 + 32 * t + 8 * (r >> 2) + 4 * hi + (r & 3);
        const float p = key < Na ? exp2f(s[t][r] * sl2 - l2) : 0.f;
        dsf[j][jj] = (__bf16)(p * (dp[t][r] - dn));
      }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int R = c0 + 32 * (j >> 1) + 16 * (j & 1) + 4 * hi;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const __bf16* p0 = sK + (R + vrow) * kXLd + 32 * t + vcol;
        const bf16x4 lo = tr_read4(p0);
        const bf16x4 up = tr_read4(p0 + 8 * kXLd);
        acc[t] = mfma32x32x16(__builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7), dsf[j],
                              acc[t]);
      }
    }
  }
  // dQ^T [D, npad] too (the dWq product's operand): lane holds column n,
  // rows h d + 32 t + 8 g + 4 hi + i; columns N .. npad - 1 get zeros
  if (n < npad) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int dd = h * kXD + 32 * t + 8 * (r >> 2) + 4 * hi + (r & 3);
        dqT[(size_t)dd * npad + n] = n_ok ? (__bf16)(acc[t][r] * scale) : (__bf16)0.f;
      }
  }
  if (!n_ok) return;
  __bf16* orow = dq + (size_t)n * D + h * kXD + 4 * hi;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 v4;
#pragma unroll
      for (int i = 0; i < 4; ++i) v4[i] = (__bf16)(acc[t][4 * g + i] * scale);
      *reinterpret_cast<bf16x4*>(orow + 32 * t + 8 * g) = v4;
    }
}

constexpr int kKW = 4;             // waves of the dK/dV kernel, 32 keys each
constexpr int kKQ = 128;           // queries per streamed tile

__global__ __launch_bounds__(64 * kKW) void xattn_bwd_dkdv_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dO, const float* __restrict__ lse,
    const float* __restrict__ delta, int N, int Na, int D, float scale, int splits,
    float* __restrict__ part_k, float* __restrict__ part_v) {
  __shared__ __align__(16) __bf16 sQ[kKQ * kXLd];
  __shared__ __align__(16) __bf16 sD[kKQ * kXLd];
  __shared__ float sL[kKQ], sDel[kKQ];
  const int split = blockIdx.x, kb = blockIdx.y, h = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int key = 128 * kb + 32 * w + l32;  // this lane's key (B operand column)
  const bool key_ok = key < Na;
  // K and V fragments of the wave's 32 keys: lane holds X[key][16 s + 8 hi .. +8]
  bf16x8 kf[8], vf[8];
  {
    const bf16x8 z = {};
    const __bf16* kr = k + (size_t)(key_ok ? key : 0) * D + h * kXD + 8 * hi;
    const __bf16* vr = v + (size_t)(key_ok ? key : 0) * D + h * kXD + 8 * hi;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      kf[s] = key_ok ? *reinterpret_cast<const bf16x8*>(kr + 16 * s) : z;
      vf[s] = key_ok ? *reinterpret_cast<const bf16x8*>(vr + 16 * s) : z;
    }
  }
  f32x16 dk[4], dv[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[t][r] = dv[t][r] = 0.f;
  const float sl2 = scale * kLog2e;
  const int G = lane >> 4, u = lane & 15;
  const int trow = u >> 2, tcol = 16 * (G & 1) + 4 * (u & 3);
  const int ntiles = (N + kKQ - 1) / kKQ;
  for (int qt = split; qt < ntiles; qt += splits) {
    const long long q0 = (long long)qt * kKQ;
    __syncthreads();
    for (int e = tid; e < kKQ * 16; e += 64 * kKW) {
      const int r = e >> 4, ch = e & 15;
      u32x4 qv = {0u, 0u, 0u, 0u}, dv4 = {0u, 0u, 0u, 0u};
      if (q0 + r < N) {
        qv = *reinterpret_cast<const u32x4*>(q + (size_t)(q0 + r) * D + h * kXD + 8 * ch);
        dv4 = *reinterpret_cast<const u32x4*>(dO + (size_t)(q0 + r) * D + h * kXD + 8 * ch);
      }
      *reinterpret_cast<u32x4*>(sQ + r * kXLd + 8 * ch) = qv;
      *reinterpret_cast<u32x4*>(sD + r * kXLd + 8 * ch) = dv4;
    }
    for (int e = tid; e < kKQ; e += 64 * kKW) {
      const bool ok = q0 + e < N;
      sL[e] = ok ? lse[(size_t)h * N + q0 + e] * kLog2e : INFINITY;  // pad rows: P = 0
      sDel[e] = ok ? delta[(size_t)h * N + q0 + e] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int qs = 0; qs < kKQ / 32; ++qs) {
      // S = Q K^T and dP = dO V^T for queries q0 + 32 qs .. +32 (rows) and the
      // wave's keys (columns): lane holds query 32 qs + 8 (r/4) + 4 hi + r%4
      f32x16 s = {}, dp = {};
      const __bf16* qr = sQ + (32 * qs + l32) * kXLd + 8 * hi;
      const __bf16* dr = sD + (32 * qs + l32) * kXLd + 8 * hi;
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        s = mfma32x32x16(*reinterpret_cast<const bf16x8*>(qr + 16 * st), kf[st], s);
        dp = mfma32x32x16(*reinterpret_cast<const bf16x8*>(dr + 16 * st), vf[st], dp);
      }
      // P and dS (bf16) in the query order of the dV / dK products: k-step j
      // (16 queries), slot jj = query 32 qs + 16 j + 8 (jj/4) + 4 hi + jj%4
      bf16x8 pf[2], dsf[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int r = 4 * (2 * j + (jj >> 2)) + (jj & 3);
          const int ql = 32 * qs + 8 * (r >> 2) + 4 * hi + (r & 3);
          const float p = key_ok ? exp2f(s[r] * sl2 - sL[ql]) : 0.f;
          const __bf16 pb = (__bf16)p;
          pf[j][jj] = pb;
          dsf[j][jj] = (__bf16)(p * (dp[r] - sDel[ql]));
        }
      // dV[key][d] += sum_q P[q][key] dO[q][d]; dK likewise with dS and Q:
      // A = P^T / dS^T (lane = key), B = dO / Q columns through transposed reads
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int R = 32 * qs + 16 * j + 4 * hi;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const __bf16* pd = sD + (R + trow) * kXLd + 32 * t + tcol;
          const __bf16* pq = sQ + (R + trow) * kXLd + 32 * t + tcol;
          const bf16x8 bd = __builtin_shufflevector(tr_read4(pd), tr_read4(pd + 8 * kXLd),
                                                    0, 1, 2, 3, 4, 5, 6, 7);
          const bf16x8 bq = __builtin_shufflevector(tr_read4(pq), tr_read4(pq + 8 * kXLd),
                                                    0, 1, 2, 3, 4, 5, 6, 7);
          dv[t] = mfma32x32x16(pf[j], bd, dv[t]);
          dk[t] = mfma32x32x16(dsf[j], bq, dk[t]);
        }
      }
    }
  }
  // lane holds X[key 128 kb + 32 w + 8 (r/4) + 4 hi + r%4][d = 32 t + l32]:
  // partial [split][h][key][d]
  const size_t hbase = ((size_t)split * gridDim.z + h) * gridDim.y * 128;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = 128 * kb + 32 * w + 8 * (r >> 2) + 4 * hi + (r & 3);
      const size_t off = (hbase + kr) * kXD + 32 * t + l32;
      part_k[off] = dk[t][r];
      part_v[off] = dv[t][r];
    }
}

// dK, dV [Na, D] bf16 = sum over splits (fixed order) of the partials; dK scaled
__global__ __launch_bounds__(256) void xattn_reduce_kernel(const float* __restrict__ part_k,
                                                           const float* __restrict__ part_v,
                                                           int splits, int heads, int kpad, int Na,
                                                           float scale, __bf16* __restrict__ dk,
                                                           __bf16* __restrict__ dv) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;  // (key, h, d)
  const long long total = (long long)Na * heads * kXD;
  if (i >= total) return;
  const int d = (int)(i % kXD);
  const int h = (int)((i / kXD) % heads);
  const int key = (int)(i / ((long long)kXD * heads));
  float sk = 0.f, sv = 0.f;
  for (int sp = 0; sp < splits; ++sp) {
    const size_t off = ((((size_t)sp * heads + h) * kpad) + key) * kXD + d;
    sk += part_k[off];
    sv += part_v[off];
  }
  dk[(size_t)key * heads * kXD + h * kXD + d] = (__bf16)(sk * scale);
  dv[(size_t)key * heads * kXD + h * kXD + d] = (__bf16)sv;
}

}  // namespace

namespace {
// the 256 x 256 kernel: operands within its 32-bit buffer offsets and K whole
// 64-deep steps
bool big_ok(int M, int N, int K, int lda, int ldb) {
  return M >= kBM && N >= kBN && K % kGK == 0 && (long long)M * lda * 2 < (1LL << 31) &&
         (long long)N * ldb * 2 < (1LL << 31);
}
int big_tiles(int M, int N) { return ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN); }
}  // namespace

hipError_t launch_gemm_nt(const __bf16* A, int lda, const __bf16* B, int ldb, int M, int N, int K,
                          void* C, int ldc, bool out_f32, bool accumulate, hipStream_t st) {
  if (big_ok(M, N, K, lda, ldb) && big_tiles(M, N) >= 128) {
    dim3 bgrid((N + kBN - 1) / kBN, (M + kBM - 1) / kBM);
    if (!out_f32)
      gemm_nt_big_kernel<false, false><<<bgrid, kBThreads, 0, st>>>(A, lda, B, ldb, M, N, K, C,
                                                                    ldc, 0);
    else if (accumulate)
      gemm_nt_big_kernel<true, true><<<bgrid, kBThreads, 0, st>>>(A, lda, B, ldb, M, N, K, C, ldc,
                                                                  0);
    else
      gemm_nt_big_kernel<true, false><<<bgrid, kBThreads, 0, st>>>(A, lda, B, ldb, M, N, K, C,
                                                                   ldc, 0);
    return hipGetLastError();
  }
  dim3 grid((N + kGN - 1) / kGN, (M + kGM - 1) / kGM);
  if (!out_f32)
    gemm_nt_kernel<false, false><<<grid, kGThreads, 0, st>>>(A, lda, B, ldb, M, N, K, C, ldc, 0);
  else if (accumulate)
    gemm_nt_kernel<true, true><<<grid, kGThreads, 0, st>>>(A, lda, B, ldb, M, N, K, C, ldc, 0);
  else
    gemm_nt_kernel<true, false><<<grid, kGThreads, 0, st>>>(A, lda, B, ldb, M, N, K, C, ldc, 0);
  return hipGetLastError();
}

namespace {
// out[m][n] = sum over z (in order) of part[z][m][n]
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int splits, int M, int N,
                                                            float* __restrict__ out) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total = (long long)M * N;
  if (i >= total) return;
  float sum = 0.f;
  for (int z = 0; z < splits; ++z) sum += part[(size_t)z * total + i];
  out[i] = sum;
}
}  // namespace

int gemm_splitk_splits(int M, int N, int K) {
  // (operand strides equal K here: the transposed token-major operands)
  const int tiles = big_ok(M, N, K, K, K) ? big_tiles(M, N)
                                          : ((M + kGM - 1) / kGM) * ((N + kGN - 1) / kGN);
  int s = (512 + tiles - 1) / tiles;
  const int kmax = (K + kGK - 1) / kGK;  // at least one k step per split
  if (s > kmax) s = kmax;
  return s < 1 ? 1 : s;
}

// fp32 C[M, N] (row stride N) = A B^T with the k range split over
// gemm_splitk_splits(M, N, K) workgroup layers; part holds splits x M x N floats.
hipError_t launch_gemm_nt_splitk(const __bf16* A, int lda, const __bf16* B, int ldb, int M, int N,
                                 int K, float* C, float* part, hipStream_t st) {
  const int splits = gemm_splitk_splits(M, N, K);
  const int kchunk = kGK * (((K + kGK - 1) / kGK + splits - 1) / splits);
  if (big_ok(M, N, K, lda, ldb)) {
    dim3 bgrid((N + kBN - 1) / kBN, (M + kBM - 1) / kBM, splits);
    gemm_nt_big_kernel<true, false><<<bgrid, kBThreads, 0, st>>>(A, lda, B, ldb, M, N, K, part,
                                                                 N, kchunk);
  } else {
    dim3 grid((N + kGN - 1) / kGN, (M + kGM - 1) / kGM, splits);
    gemm_nt_kernel<true, false><<<grid, kGThreads, 0, st>>>(A, lda, B, ldb, M, N, K, part, N,
                                                            kchunk);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  splitk_reduce_kernel<<<(unsigned)(((long long)M * N + 255) / 256), 256, 0, st>>>(part, splits, M,
                                                                                N, C);
  return hipGetLastError();
}

hipError_t launch_transpose(const __bf16* src, int R, int Cc, int lds, __bf16* dst, int ldo,
                            hipStream_t st) {
  // every caller passes C, D (multiples of 64) or padded token counts and 16-byte aligned rows
  if (((lds | ldo | Cc) & 7) != 0 || (((uintptr_t)src | (uintptr_t)dst) & 15) != 0)
    return hipErrorInvalidValue;
  dim3 grid((Cc + 63) / 64, (ldo + 255) / 256);
  transpose16_kernel<<<grid, 256, 0, st>>>(src, R, Cc, lds, dst, ldo);
  return hipGetLastError();
}

int xattn_na_pad(int n_audio) { return 64 * ((n_audio + 63) / 64); }

hipError_t launch_xattn_fwd(int N, int Na, int heads, const __bf16* x, const __bf16* a, int C,
                            const __bf16* wq, const __bf16* wk, const __bf16* wv,
                            const __bf16* wo, __bf16* q, __bf16* k, __bf16* v, __bf16* o,
                            float* lse, __bf16* y, hipStream_t st) {
  const int D = heads * kXD;
  hipError_t e = launch_gemm_nt(x, C, wq, C, N, D, C, q, D, false, false, st);
  if (e == hipSuccess) e = launch_gemm_nt(a, C, wk, C, Na, D, C, k, D, false, false, st);
  if (e == hipSuccess) e = launch_gemm_nt(a, C, wv, C, Na, D, C, v, D, false, false, st);
  if (e != hipSuccess) return e;
  const int na_pad = xattn_na_pad(Na);
  if (na_pad > kXMaxNa) return hipErrorInvalidValue;
  dim3 grid((N + kXQ - 1) / kXQ, heads);
  xattn_fwd_kernel<<<grid, 64 * kXWaves, 0, st>>>(q, k, v, N, Na, na_pad, D,
                                                  kLog2e / sqrtf((float)kXD), o, lse);
  e = hipGetLastError();
  if (e == hipSuccess) e = launch_gemm_nt(o, D, wo, D, N, C, D, y, C, false, false, st);
  return e;
}

namespace {
size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }
int up64(int x) { return 64 * ((x + 63) / 64); }

// Backward workspace, in order: dO, dQ [N, D] bf16 | dK, dV [Na, D] bf16 |
// delta [H, N] f32 | dK, dV partials [splits, H, kpad, 128] f32 | Wo^T [D, C],
// Wq^T, Wk^T, Wv^T [C, D] bf16 | dY^T, X^T [C, Npad], O^T, dQ^T [D, Npad] bf16 |
// A^T [C, Nap], dK^T, dV^T [D, Nap] bf16 | split-K partials of the weight
// gradients over the tokens [ksplits, C D] f32.
struct XBwdWs {
  int splits, kpad, npad, nap, ksplits;
  size_t off[20];
  size_t total;
};

XBwdWs xattn_bwd_layout(int N, int Na, int C, int heads) {
  XBwdWs w{};
  const int D = heads * kXD;
  w.kpad = 128 * ((Na + 127) / 128);
  const int kblocks = w.kpad / 128;
  const int ntiles = (N + kKQ - 1) / kKQ;
  // query splits of the dK/dV pass: as many as keep every (split, key block,
  // head) workgroup resident at once (two per CU by LDS, 512 on 256 CUs);
  // one more and the excess would run as a second, nearly empty round
  w.splits = 512 / (heads * kblocks);
  if (w.splits > ntiles) w.splits = ntiles;
  if (w.splits < 1) w.splits = 1;
  w.npad = up64(N);
  w.nap = up64(Na);
  w.ksplits = std::max(gemm_splitk_splits(C, D, w.npad), gemm_splitk_splits(D, C, w.npad));
  const size_t b2 = sizeof(__bf16);
  const size_t sizes[] = {
      (size_t)N * D * b2, (size_t)N * D * b2, (size_t)Na * D * b2, (size_t)Na * D * b2,
      (size_t)heads * N * 4,
      (size_t)w.splits * heads * w.kpad * kXD * 4, (size_t)w.splits * heads * w.kpad * kXD * 4,
      (size_t)D * C * b2, (size_t)C * D * b2, (size_t)C * D * b2, (size_t)C * D * b2,
      (size_t)C * w.npad * b2, (size_t)C * w.npad * b2, (size_t)D * w.npad * b2,
      (size_t)D * w.npad * b2,
      (size_t)C * w.nap * b2, (size_t)D * w.nap * b2, (size_t)D * w.nap * b2,
      (size_t)w.ksplits * C * D * 4};
  size_t o = 0;
  for (int i = 0; i < (int)(sizeof(sizes) / sizeof(sizes[0])); ++i) {
    w.off[i] = o;
    o += al256(sizes[i]);
  }
  w.total = o;
  return w;
}
}  // namespace

size_t xattn_bwd_workspace(int N, int Na, int C, int heads) {
  return xattn_bwd_layout(N, Na, C, heads).total;
}

hipError_t launch_xattn_bwd(int N, int Na, int heads, const __bf16* x, const __bf16* a, int C,
                            const __bf16* wq, const __bf16* wk, const __bf16* wv,
                            const __bf16* wo, const __bf16* q, const __bf16* k, const __bf16* v,
                            const __bf16* o, const float* lse, const __bf16* dy, float* dx,
                            float* da, float* dwq, float* dwk, float* dwv, float* dwo, void* ws,
                            hipStream_t st) {
  const int D = heads * kXD;
  const XBwdWs w = xattn_bwd_layout(N, Na, C, heads);
  char* base = static_cast<char*>(ws);
  auto bf = [&](int i) { return reinterpret_cast<__bf16*>(base + w.off[i]); };
  auto f32 = [&](int i) { return reinterpret_cast<float*>(base + w.off[i]); };
  __bf16 *dO = bf(0), *dQ = bf(1), *dK = bf(2), *dV = bf(3);
  float *delta = f32(4), *pk = f32(5), *pv = f32(6);
  __bf16 *woT = bf(7), *wqT = bf(8), *wkT = bf(9), *wvT = bf(10);
  __bf16 *dyT = bf(11), *xT = bf(12), *oT = bf(13), *dqT = bf(14);
  __bf16 *aT = bf(15), *dkT = bf(16), *dvT = bf(17);
  float* kpart = f32(18);
  const float scale = 1.f / sqrtf((float)kXD);
  hipError_t e = hipSuccess;
#define BSA_X(call)                 \
  do {                              \
    e = (call);                     \
    if (e != hipSuccess) return e;  \
  } while (0)
  // dO = dY Wo
  BSA_X(launch_transpose(wo, C, D, D, woT, C, st));
  BSA_X(launch_gemm_nt(dy, C, woT, C, N, D, C, dO, D, false, false, st));
  // D = rowsum(dO * O); dQ; dK, dV
  xattn_delta_kernel<<<(unsigned)(((long long)N * heads * 16 + 255) / 256), 256, 0, st>>>(
      dO, o, N, heads, delta);
  BSA_X(hipGetLastError());
  const int na_pad = xattn_na_pad(Na);
  xattn_bwd_dq_kernel<<<dim3((N + kXQ - 1) / kXQ, heads), 64 * kXWaves, 0, st>>>(
      q, k, v, dO, lse, delta, N, Na, na_pad, D, scale, dQ, dqT, w.npad);
  BSA_X(hipGetLastError());
  xattn_bwd_dkdv_kernel<<<dim3(w.splits, w.kpad / 128, heads), 64 * kKW, 0, st>>>(
      q, k, v, dO, lse, delta, N, Na, D, scale, w.splits, pk, pv);
  BSA_X(hipGetLastError());
  xattn_reduce_kernel<<<(unsigned)(((long long)Na * D + 255) / 256), 256, 0, st>>>(
      pk, pv, w.splits, heads, w.kpad, Na, scale, dK, dV);
  BSA_X(hipGetLastError());
  // dWo = dY^T O
  BSA_X(launch_transpose(dy, N, C, C, dyT, w.npad, st));
  BSA_X(launch_transpose(o, N, D, D, oT, w.npad, st));
  BSA_X(launch_gemm_nt_splitk(dyT, w.npad, oT, w.npad, C, D, w.npad, dwo, kpart, st));
  // dX = dQ Wq, dWq = dQ^T X
  BSA_X(launch_transpose(wq, D, C, C, wqT, D, st));
  BSA_X(launch_gemm_nt(dQ, D, wqT, D, N, C, D, dx, C, true, false, st));
  BSA_X(launch_transpose(x, N, C, C, xT, w.npad, st));
  BSA_X(launch_gemm_nt_splitk(dqT, w.npad, xT, w.npad, D, C, w.npad, dwq, kpart, st));
  // dA = dK Wk + dV Wv, dWk = dK^T A, dWv = dV^T A
  BSA_X(launch_transpose(wk, D, C, C, wkT, D, st));
  BSA_X(launch_transpose(wv, D, C, C, wvT, D, st));
  BSA_X(launch_gemm_nt(dK, D, wkT, D, Na, C, D, da, C, true, false, st));
  BSA_X(launch_gemm_nt(dV, D, wvT, D, Na, C, D, da, C, true, true, st));
  BSA_X(launch_transpose(a, Na, C, C, aT, w.nap, st));
  BSA_X(launch_transpose(dK, Na, D, D, dkT, w.nap, st));
  BSA_X(launch_transpose(dV, Na, D, D, dvT, w.nap, st));
  BSA_X(launch_gemm_nt(dkT, w.nap, aT, w.nap, D, C, w.nap, dwk, C, true, false, st));
  BSA_X(launch_gemm_nt(dvT, w.nap, aT, w.nap, D, C, w.nap, dwv, C, true, false, st));
#undef BSA_X
  return hipSuccess;
}

}  // namespace bsa

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
//  transpose_kernel  bf16 [R, Cc] -> [Cc, ldo] through LDS, columns R..ldo-1
//                    zero (so transposed rows are whole 16-byte chunks).
//  xattn_fwd_kernel  per (256 queries, head): K_h, V_h of every audio token in
//                    LDS; per wave 32 queries, S^T = K Q^T and O^T += V^T P^T on
//                    MFMA over 64-key chunks with an online softmax; writes O
//                    (bf16) and lse (natural log, fp32).
#include <math.h>

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

template <bool kOutF32, bool kAccum>
__global__ __launch_bounds__(kGThreads) void gemm_nt_kernel(const __bf16* __restrict__ A, int lda,
                                                          const __bf16* __restrict__ B, int ldb,
                                                          int M, int N, int K, void* C, int ldc) {
  __shared__ __align__(16) __bf16 sA[2][kGM * kGK];
  __shared__ __align__(16) __bf16 sB[2][kGN * kGK];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int m0 = blockIdx.y * kGM, n0 = blockIdx.x * kGN;
  const int wm = w >> 1, wn = w & 1;
  // loader: chunk e = tid + 256 u (u = 0..3) of a tile: row e / 8, chunk e % 8
  u32x4 ra[4], rb[4];
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  auto gload = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + kGThreads * u, r = e >> 3, ch = e & 7;
      const int k = k0 + 8 * ch;
      ra[u] = (m0 + r < M && k < K)
                  ? *reinterpret_cast<const u32x4*>(A + (size_t)(m0 + r) * lda + k) : z4;
      rb[u] = (n0 + r < N && k < K)
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
  const int nk = (K + kGK - 1) / kGK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * kGK);
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

// -------------------------------------------------------------- transpose --
__global__ __launch_bounds__(256) void transpose_kernel(const __bf16* __restrict__ src, int R,
                                                        int Cc, int lds, __bf16* __restrict__ dst,
                                                        int ldo) {
  __shared__ __bf16 t[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64, tid = threadIdx.x;
  for (int e = tid; e < 64 * 64; e += 256) {
    const int r = e >> 6, c = e & 63;
    t[r][c] = (r0 + r < R && c0 + c < Cc) ? src[(size_t)(r0 + r) * lds + c0 + c] : (__bf16)0.f;
  }
  __syncthreads();
  for (int e = tid; e < 64 * 64; e += 256) {
    const int c = e >> 6, r = e & 63;  // dst row c0 + c, column r0 + r
    if (c0 + c < Cc && r0 + r < ldo) dst[(size_t)(c0 + c) * ldo + r0 + r] = t[r][c];
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

}  // namespace

hipError_t launch_gemm_nt(const __bf16* A, int lda, const __bf16* B, int ldb, int M, int N, int K,
                          void* C, int ldc, bool out_f32, bool accumulate, hipStream_t st) {
  dim3 grid((N + kGN - 1) / kGN, (M + kGM - 1) / kGM);
  if (!out_f32)
    gemm_nt_kernel<false, false><<<grid, kGThreads, 0, st>>>(A, lda, B, ldb, M, N, K, C, ldc);
  else if (accumulate)
    gemm_nt_kernel<true, true><<<grid, kGThreads, 0, st>>>(A, lda, B, ldb, M, N, K, C, ldc);
  else
    gemm_nt_kernel<true, false><<<grid, kGThreads, 0, st>>>(A, lda, B, ldb, M, N, K, C, ldc);
  return hipGetLastError();
}

hipError_t launch_transpose(const __bf16* src, int R, int Cc, int lds, __bf16* dst, int ldo,
                            hipStream_t st) {
  dim3 grid((Cc + 63) / 64, (ldo + 63) / 64);
  transpose_kernel<<<grid, 256, 0, st>>>(src, R, Cc, lds, dst, ldo);
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

}  // namespace bsa

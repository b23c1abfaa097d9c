// Zone scoring and block-shape choice.
//
// Prism page (trawling.dev/post/2299), section on block composition matched to
// regional information: per macro-zone, the channel-wise variance of the video
// features (how fast and along which direction content changes) and the
// feature norm of the audio-to-video cross-attention (how strongly audio drives
// the region) together set the zone's block shape; fast-changing or strongly
// coupled axes are split more finely. Reading implemented (no formula on the
// page): one A2V head with identity projections and scale 1/sqrt(C),
//   g_n = || sum_j p_nj A_j ||,  p_n = softmax_j(X_n . A_j / sqrt(C)),
// per-axis within-line variances of X (averaged over channels) and of g, each
// normalised by its mean over non-empty (zone, axis) pairs, and the shape that
// minimises the predicted within-block variance sum_a r_a (b_a^2-1)/(Z_a^2-1).
//
// Kernels:
//  gram_kernel     G = A A^T (fp64 accumulation, stored fp32), tiny.
//  a2v_kernel      per 128 tokens: logits^T = A X^T on bf16 MFMA (exact products,
//                  fp32 sums), softmax in fp32 registers (lane-local rows), then
//                  g^2 = p^T G p as Y = G P^T on fp32 MFMA (32x32x2) and a
//                  lane-local dot with P. Writes g [N] fp32.
//  line_kernel     per (zone, 32-channel chunk): the zone's slice is staged in
//                  LDS, then sum x^2 and the squared line sums along t, h, w in
//                  fp64 (bf16 inputs make these sums exact), so
//                  V_a = (sum x^2 - sum_lines S^2/len) / (C n_z).
//                  The same kernel with one channel handles g.
//  decide_kernel   one workgroup: reduce the partials in a fixed order, the
//                  means, r, the costs and the tie rule; writes the shape ids.
#include <math.h>

#include "attn_common.hpp"
#include "kernels.hpp"

namespace bsa {
namespace {

constexpr double kTieRel = 1e-6;

// ------------------------------------------------------------- Gram matrix --
__global__ __launch_bounds__(256) void gram_kernel(const __bf16* A, int Na, int na_pad, int C,
                                                   float* gram) {
  const int j = blockIdx.x;  // row
  for (int k = threadIdx.x; k < na_pad; k += 256) {
    double s = 0.0;
    if (j < Na && k < Na)
      for (int c = 0; c < C; ++c)
        s += (double)(float)A[(size_t)j * C + c] * (double)(float)A[(size_t)k * C + c];
    gram[(size_t)j * na_pad + k] = (float)s;
  }
}

// --------------------------------------------------------------- A2V norm --
constexpr int kTok = 128;        // tokens per workgroup (4 waves x 32)
constexpr int kCh = 64;          // channels per LDS stage
constexpr int kXS = kCh + 8;     // LDS row stride (bf16 elements)
constexpr int kMaxMT = 8;        // audio tiles of 32 (n_audio <= 256)

template <int MT>
__global__ __launch_bounds__(256) void a2v_kernel(const __bf16* X, int C, long long N,
                                                  const __bf16* A, int Na, const float* gram,
                                                  float inv_sqrt_c, float* gout) {
  __shared__ __align__(16) __bf16 xs[kTok * kXS];
  __shared__ __align__(16) __bf16 as[32 * MT * kXS];
  __shared__ float gs[32 * (32 * MT + 1)];
  constexpr int NA_PAD = 32 * MT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const long long n0 = (long long)blockIdx.x * kTok;

  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;

  for (int c0 = 0; c0 < C; c0 += kCh) {
    __syncthreads();
    for (int e = tid; e < kTok * (kCh / 8); e += 256) {
      const int r = e >> 3, c = e & 7;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (n0 + r < N) v = *reinterpret_cast<const uint4*>(X + (size_t)(n0 + r) * C + c0 + 8 * c);
      *reinterpret_cast<uint4*>(xs + r * kXS + 8 * c) = v;
    }
    for (int e = tid; e < NA_PAD * (kCh / 8); e += 256) {
      const int r = e >> 3, c = e & 7;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r < Na) v = *reinterpret_cast<const uint4*>(A + (size_t)r * C + c0 + 8 * c);
      *reinterpret_cast<uint4*>(as + r * kXS + 8 * c) = v;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kCh / 16; ++ks) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(xs + (32 * w + l32) * kXS + 16 * ks + 8 * hi);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(as + (32 * mt + l32) * kXS + 16 * ks + 8 * hi);
        acc[mt] = mfma32x32x16(a, b, acc[mt]);
      }
    }
  }

  // softmax over the audio axis; lane holds audio 32mt + 8(r/4) + 4hi + r%4
  float mx = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int a = 32 * mt + 8 * (r >> 2) + 4 * hi + (r & 3);
      if (a < Na) mx = fmaxf(mx, acc[mt][r]);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  float z = 0.f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int a = 32 * mt + 8 * (r >> 2) + 4 * hi + (r & 3);
      const float p = a < Na ? expf((acc[mt][r] - mx) * inv_sqrt_c) : 0.f;
      acc[mt][r] = p;
      z += p;
    }
  z += __shfl_xor(z, 32);

  // g^2 * z^2 = sum_m p_m (G p)_m, with (G p) from fp32 MFMA per 32-row tile of G
  float gsq = 0.f;
  for (int mt = 0; mt < MT; ++mt) {
    __syncthreads();
    for (int e = tid; e < 32 * NA_PAD; e += 256) {
      const int r = e / NA_PAD, c = e % NA_PAD;
      gs[r * (NA_PAD + 1) + c] = gram[(size_t)(32 * mt + r) * NA_PAD + c];
    }
    __syncthreads();
    f32x16 y;
#pragma unroll
    for (int r = 0; r < 16; ++r) y[r] = 0.f;
#pragma unroll
    for (int kt = 0; kt < MT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int a = 32 * kt + 8 * (r >> 2) + 4 * hi + (r & 3);
        y = __builtin_amdgcn_mfma_f32_32x32x2f32(gs[l32 * (NA_PAD + 1) + a], acc[kt][r], y, 0, 0, 0);
      }
#pragma unroll
    for (int r = 0; r < 16; ++r) gsq = fmaf(y[r], acc[mt][r], gsq);
  }
  gsq += __shfl_xor(gsq, 32);
  const long long n = n0 + 32 * w + l32;
  if (hi == 0 && n < N) gout[n] = sqrtf(fmaxf(gsq, 0.f)) / z;
}

// ------------------------------------------------------- line sum partials --
// Partials per (zone, chunk of kLC channels): [0] sum x^2, [1..3] sum over the
// lines along t, h, w of (line sum)^2 / line length, all in fp64 (bf16 and fp32
// inputs make these sums exact). The zone's slice of kLC channels is staged in
// LDS with 16-byte loads, then each line is summed by one thread (no atomics,
// fixed summation order).
constexpr int kLC = 32;  // channels per workgroup

template <typename T>
__global__ __launch_bounds__(256) void line_kernel(Lay L, const T* __restrict__ X, int C,
                                                   double* __restrict__ part) {
  __shared__ T xs[4 * 16 * 16 * kLC];  // [t][h][w][c]: 64 KB for bf16 (exact copies)
  __shared__ double red[4][4];
  const int z = blockIdx.x, chunk = blockIdx.y, nchunks = gridDim.y;
  const int zzt = z / (L.gzh * L.gzw), zzh = (z / L.gzw) % L.gzh, zzw = z % L.gzw;
  const int t0 = zzt * L.zt, h0 = zzh * L.zh, w0 = zzw * L.zw;
  const int vt = imax(0, imin(L.zt, L.T - t0));
  const int vh = imax(0, imin(L.zh, L.H - h0));
  const int vw = imax(0, imin(L.zw, L.W - w0));
  const int c0 = chunk * kLC;
  const int cw = imin(kLC, C - c0);            // channels in this chunk
  constexpr int EPC = 16 / sizeof(T);          // elements per 16-byte load
  const int nseg = kLC / EPC;                  // 16-byte segments per token
  const int ntok = vt * vh * vw;
  // stage: token k (raster inside the zone's real box), segment sg
  for (int e = threadIdx.x; e < ntok * nseg; e += 256) {
    const int k = e / nseg, sg = e - k * nseg;
    const int tw = k % vw, th = (k / vw) % vh, tt = k / (vw * vh);
    const long long n = ((long long)(t0 + tt) * L.H + (h0 + th)) * L.W + (w0 + tw);
    T* dst = xs + ((tt * 16 + th) * 16 + tw) * kLC + sg * EPC;
    const int cc = c0 + sg * EPC;
    if (cc + EPC <= C && (C % EPC) == 0) {
      *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(X + n * C + cc);
    } else {
      for (int q = 0; q < EPC; ++q) dst[q] = cc + q < C ? X[n * C + cc + q] : (T)0.f;
    }
  }
  __syncthreads();
  double q = 0.0, rt = 0.0, rh = 0.0, rw = 0.0;
  // w-lines (t, h, c) and the squares
  for (int e = threadIdx.x; e < vt * vh * cw; e += 256) {
    const int c = e % cw, th = (e / cw) % vh, tt = e / (cw * vh);
    const T* p = xs + ((tt * 16 + th) * 16) * kLC + c;
    double sum = 0.0;
    for (int tw = 0; tw < vw; ++tw) {
      const double x = (double)(float)p[tw * kLC];
      sum += x;
      q += x * x;
    }
    rw += sum * sum / (double)vw;
  }
  // h-lines (t, w, c)
  for (int e = threadIdx.x; e < vt * vw * cw; e += 256) {
    const int c = e % cw, tw = (e / cw) % vw, tt = e / (cw * vw);
    const T* p = xs + (tt * 16 * 16 + tw) * kLC + c;
    double sum = 0.0;
    for (int th = 0; th < vh; ++th) sum += (double)(float)p[th * 16 * kLC];
    rh += sum * sum / (double)vh;
  }
  // t-lines (h, w, c)
  for (int e = threadIdx.x; e < vh * vw * cw; e += 256) {
    const int c = e % cw, tw = (e / cw) % vw, th = e / (cw * vw);
    const T* p = xs + (th * 16 + tw) * kLC + c;
    double sum = 0.0;
    for (int tt = 0; tt < vt; ++tt) sum += (double)(float)p[tt * 16 * 16 * kLC];
    rt += sum * sum / (double)vt;
  }
  // workgroup reduction in a fixed order (deterministic)
  double vals[4] = {q, rt, rh, rw};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    double v = vals[k];
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if ((threadIdx.x & 63) == 0) red[k][threadIdx.x >> 6] = v;
  }
  __syncthreads();
  if (threadIdx.x < 4) {
    const double sres = red[threadIdx.x][0] + red[threadIdx.x][1] + red[threadIdx.x][2] +
                        red[threadIdx.x][3];
    part[((size_t)z * nchunks + chunk) * 4 + threadIdx.x] = sres;
  }
}

// ------------------------------------------------------------------ decide --
__global__ __launch_bounds__(256) void decide_kernel(Lay L, int C, int nchunks,
                                                     const double* xpart, const double* gpart,
                                                     int use_audio, int32_t* zone_shape,
                                                     double* zone_stats, double* scratch) {
  // scratch: V [nZ][3], G [nZ][3], nz [nZ]
  double* V = scratch;
  double* G = scratch + 3 * L.nZ;
  double* NZ = scratch + 6 * L.nZ;
  __shared__ double sv[256], sg[256];
  __shared__ int scount[256];
  const int tid = threadIdx.x;
  double accv = 0.0, accg = 0.0;
  int cnt = 0;
  for (int z = tid; z < L.nZ; z += 256) {
    const int zzt = z / (L.gzh * L.gzw), zzh = (z / L.gzw) % L.gzh, zzw = z % L.gzw;
    const int vt = imax(0, imin(L.zt, L.T - zzt * L.zt));
    const int vh = imax(0, imin(L.zh, L.H - zzh * L.zh));
    const int vw = imax(0, imin(L.zw, L.W - zzw * L.zw));
    const double nz = (double)vt * vh * vw;
    NZ[z] = nz;
    double q = 0.0, r[3] = {0.0, 0.0, 0.0};
    for (int k = 0; k < nchunks; ++k) {
      const double* p = xpart + ((size_t)z * nchunks + k) * 4;
      q += p[0];
      r[0] += p[1];
      r[1] += p[2];
      r[2] += p[3];
    }
    for (int a = 0; a < 3; ++a) {
      V[3 * z + a] = nz > 0 ? (q - r[a]) / ((double)C * nz) : 0.0;
      G[3 * z + a] = (use_audio && nz > 0) ? (gpart[4 * z] - gpart[4 * z + 1 + a]) / nz : 0.0;
    }
    if (nz > 0) {
      accv += V[3 * z] + V[3 * z + 1] + V[3 * z + 2];
      accg += G[3 * z] + G[3 * z + 1] + G[3 * z + 2];
      cnt += 3;
    }
  }
  sv[tid] = accv;
  sg[tid] = accg;
  scount[tid] = cnt;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) {
      sv[tid] += sv[tid + s];
      sg[tid] += sg[tid + s];
      scount[tid] += scount[tid + s];
    }
    __syncthreads();
  }
  const double vbar = scount[0] ? sv[0] / scount[0] : 0.0;
  const double gbar = scount[0] ? sg[0] / scount[0] : 0.0;
  for (int z = tid; z < L.nZ; z += 256) {
    double r[3];
    for (int a = 0; a < 3; ++a) {
      r[a] = 0.0;
      if (NZ[z] > 0) {
        if (vbar > 0) r[a] += V[3 * z + a] / vbar;
        if (use_audio && gbar > 0) r[a] += G[3 * z + a] / gbar;
      }
    }
    double cost[4];
    double cmin = INFINITY;
    for (int s = 0; s < L.n_shapes; ++s) {
      cost[s] = 0.0;
      for (int a = 0; a < 3; ++a) {
        const int Z = a == 0 ? L.zt : (a == 1 ? L.zh : L.zw);
        const int b = L.sh[s][a];
        const double f = Z == 1 ? 0.0 : (double)(b * b - 1) / (double)(Z * Z - 1);
        cost[s] += r[a] * f;
      }
      cmin = fmin(cmin, cost[s]);
    }
    int pick = 0;
    for (int s = L.n_shapes - 1; s >= 0; --s)
      if (cost[s] <= cmin + kTieRel * cmin) pick = s;
    zone_shape[z] = pick;
    if (zone_stats) {
      for (int a = 0; a < 3; ++a) {
        zone_stats[6 * z + 2 * a] = V[3 * z + a];
        zone_stats[6 * z + 2 * a + 1] = G[3 * z + a];
      }
    }
  }
}

__global__ void fill_zero_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// Workspace: g [N] f32 | gram [pad^2] f32 | xpart [nZ][chunks][4] | gpart [nZ][4] | scratch [7 nZ]
size_t zone_score_workspace(const Lay& L, int C, int n_audio) {
  const int pad = 32 * ((n_audio + 31) / 32);
  const int chunks = (C + kLC - 1) / kLC;
  return al256((size_t)L.N * sizeof(float)) + al256((size_t)pad * pad * sizeof(float)) +
         al256((size_t)L.nZ * chunks * 4 * sizeof(double)) +
         al256((size_t)L.nZ * 4 * sizeof(double)) + al256((size_t)L.nZ * 7 * sizeof(double));
}

hipError_t launch_zone_score(const Lay& L, const void* video, int C, const void* audio,
                             int n_audio, int32_t* zone_shape, double* zone_stats, void* ws,
                             hipStream_t st) {
  if (L.n_shapes == 1 || video == nullptr) {  // fixed layout: one shape everywhere
    fill_zero_kernel<<<(L.nZ + 255) / 256, 256, 0, st>>>(zone_shape, L.nZ);
    return hipGetLastError();
  }
  const int pad = 32 * ((n_audio + 31) / 32);
  const int chunks = (C + kLC - 1) / kLC;
  char* p = static_cast<char*>(ws);
  float* g = reinterpret_cast<float*>(p);
  p += al256((size_t)L.N * sizeof(float));
  float* gram = reinterpret_cast<float*>(p);
  p += al256((size_t)pad * pad * sizeof(float));
  double* xpart = reinterpret_cast<double*>(p);
  p += al256((size_t)L.nZ * chunks * 4 * sizeof(double));
  double* gpart = reinterpret_cast<double*>(p);
  p += al256((size_t)L.nZ * 4 * sizeof(double));
  double* scratch = reinterpret_cast<double*>(p);

  const __bf16* X = static_cast<const __bf16*>(video);
  const bool use_audio = audio != nullptr && n_audio > 0;
  if (use_audio) {
    const __bf16* A = static_cast<const __bf16*>(audio);
    gram_kernel<<<pad, 256, 0, st>>>(A, n_audio, pad, C, gram);
    const unsigned grid = (unsigned)((L.N + kTok - 1) / kTok);
    const float isc = 1.0f / sqrtf((float)C);
    switch (pad / 32) {
#define BSA_A2V(MT) \
  case MT: a2v_kernel<MT><<<grid, 256, 0, st>>>(X, C, L.N, A, n_audio, gram, isc, g); break;
      BSA_A2V(1) BSA_A2V(2) BSA_A2V(3) BSA_A2V(4) BSA_A2V(5) BSA_A2V(6) BSA_A2V(7) BSA_A2V(8)
#undef BSA_A2V
      default: return hipErrorInvalidValue;
    }
    line_kernel<float><<<dim3(L.nZ, 1), 256, 0, st>>>(L, g, 1, gpart);
  }
  line_kernel<__bf16><<<dim3(L.nZ, chunks), 256, 0, st>>>(L, X, C, xpart);
  decide_kernel<<<1, 256, 0, st>>>(L, C, chunks, xpart, gpart, use_audio ? 1 : 0, zone_shape,
                                   zone_stats, scratch);
  return hipGetLastError();
}

}  // namespace bsa

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
//  gram_kernel     G = A A^T on bf16 MFMA (exact products, fp32 sums), tiny;
//                  the upper tile pairs, stored in fp32 MFMA operand order.
//  a2v_kernel      per 256 tokens: logits^T = A X^T on bf16 MFMA (exact products,
//                  fp32 sums), softmax in fp32 registers (lane-local rows), then
//                  g^2 = p^T G p as Y = G P^T on fp32 MFMA (32x32x2) over the
//                  upper tile pairs of the symmetric G and a lane-local dot
//                  with P. Writes g [N] fp32.
//  line_kernel     per (zone, 32-channel chunk): the zone is streamed through
//                  LDS one t-slice at a time; sum x^2 and the squared line sums
//                  along t, h, w in fp64 (bf16 inputs make these sums exact), so
//                  V_a = (sum x^2 - sum_lines S^2/len) / (C n_z).
//                  The same kernel with one channel handles g.
//  decide_kernel   one workgroup: reduce the partials in a fixed order, the
//                  means, r, the costs and the tie rule; writes the shape ids.
#include <math.h>

#include <type_traits>

#include "attn_common.hpp"
#include "kernels.hpp"

namespace bsa {
namespace {

constexpr double kTieRel = 1e-6;

// ------------------------------------------------------------- Gram matrix --
// One wavefront per tile pair (mt, kt), kt >= mt, of G = A A^T on bf16 MFMA
// (the products of bf16 values are exact and accumulate in fp32; rows past Na
// read as zero). The tile is stored in the operand order the A2V kernel's
// fp32 MFMA takes: lane l = 32 hi + l32 of pair p owns 16 consecutive floats,
// float r = G[32 mt + l32][32 kt + 8 (r / 4) + 4 hi + r % 4]. The MFMA result
// of rows kt x columns mt has exactly that lane layout (G is symmetric, and
// G[i][j], G[j][i] are the same products summed in the same order).
__host__ __device__ constexpr int gram_pairs(int mt_count) { return mt_count * (mt_count + 1) / 2; }

__global__ __launch_bounds__(64) void gram_kernel(const __bf16* A, int Na, int mt_count, int C,
                                                  float* gsw) {
  const int p = blockIdx.x, lane = threadIdx.x;
  int mt = 0, rem = p;
  while (rem >= mt_count - mt) rem -= mt_count - mt++;
  const int kt = mt + rem;
  const int l32 = lane & 31, hi = lane >> 5;
  const int ra = 32 * kt + l32, rb = 32 * mt + l32;
  const __bf16* pa = A + (size_t)ra * C + 8 * hi;
  const __bf16* pb = A + (size_t)rb * C + 8 * hi;
  f32x16 acc = {};
  const bf16x8 zero = {};
  for (int c = 0; c < C; c += 64) {
    bf16x8 a[4], b[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {  // C is a multiple of 64
      a[s] = ra < Na ? *reinterpret_cast<const bf16x8*>(pa + c + 16 * s) : zero;
      b[s] = rb < Na ? *reinterpret_cast<const bf16x8*>(pb + c + 16 * s) : zero;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma32x32x16(a[s], b[s], acc);
  }
  float4* out = reinterpret_cast<float4*>(gsw + ((size_t)p * 64 + lane) * 16);
#pragma unroll
  for (int v = 0; v < 4; ++v)
    out[v] = make_float4(acc[4 * v], acc[4 * v + 1], acc[4 * v + 2], acc[4 * v + 3]);
}

// --------------------------------------------------------------- A2V norm --
// 8 wavefronts x 32 tokens per workgroup. Phase 1, logits^T = A X^T on bf16
// MFMA: X fragments are loaded straight into registers (each token row is read
// once, by its own wavefront) one channel chunk ahead; A, shared by the
// wavefronts, streams through LDS in 64-channel chunks, double-buffered, with
// hand-issued buffer loads (rows past Na read as zero) laid out piece-major
// ([8-channel piece][audio row]) so the fragment reads are conflict free.
// Phase 2: softmax in fp32 registers, then g^2 z^2 = p^T G p on fp32 MFMA over
// the tile pairs kt >= mt of the symmetric G (off-diagonal pairs counted twice),
// each pair's G operands read from the operand-ordered copy the Gram kernel
// writes, straight into registers, one pair ahead.
constexpr int kA2vWaves = 8;
constexpr int kTok = 32 * kA2vWaves;  // tokens per workgroup
constexpr int kCh = 64;               // channels per A chunk

template <int MT>
__global__ __launch_bounds__(64 * kA2vWaves) void a2v_kernel(const __bf16* X, int C, long long N,
                                                             const __bf16* A, int Na,
                                                             const float* gsw, float inv_sqrt_c,
                                                             float* gout) {
  constexpr int NA_PAD = 32 * MT;
  constexpr int SLOTS = 8 * NA_PAD;               // 16-byte slots per A chunk
  constexpr int ABUF = SLOTS * 8;                  // bf16 elements per A buffer
  __shared__ __align__(16) __bf16 abuf[2 * ABUF];  // [2][piece][row][8]
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const long long n0 = (long long)blockIdx.x * kTok + 32 * w;  // this wave's first token
  const long long tok = n0 + l32;
  const bool tok_ok = tok < N;
  const int nchunks = C / kCh;

  // A chunk ch: LDS slot s = piece * NA_PAD + row <- A[row][64 ch + 8 piece ..]
  // (zero for rows past Na); thread tid stages slots tid + 512 j.
  constexpr int kAJ = (SLOTS + 64 * kA2vWaves - 1) / (64 * kA2vWaves);
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  auto load_a = [&](int ch, u32x4 (&ar)[kAJ]) {
#pragma unroll
    for (int j = 0; j < kAJ; ++j) {
      const int sl = tid + 64 * kA2vWaves * j;
      const int piece = sl / NA_PAD, r = sl - piece * NA_PAD;
      ar[j] = (sl < SLOTS && r < Na)
                  ? *reinterpret_cast<const u32x4*>(A + (size_t)r * C + kCh * ch + 8 * piece)
                  : zero4;
    }
  };
  auto store_a = [&](const u32x4 (&ar)[kAJ], int bf) {
#pragma unroll
    for (int j = 0; j < kAJ; ++j) {
      const int sl = tid + 64 * kA2vWaves * j;
      if (sl < SLOTS) *reinterpret_cast<u32x4*>(abuf + bf * ABUF + sl * 8) = ar[j];
    }
  };
  // X fragments of chunk ch: lane holds X[tok][64 ch + 16 ks + 8 hi .. +8]
  // (tokens past N read the last token; their results are not written)
  const long long tokc = tok_ok ? tok : N - 1;
  auto load_x = [&](int ch, bf16x8 (&xf)[4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      xf[ks] = *reinterpret_cast<const bf16x8*>(X + tokc * C + kCh * ch + 16 * ks + 8 * hi);
  };

  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;

  // Pipeline: X fragments three chunks ahead (a ring of four register sets),
  // A one chunk ahead in registers and one more in LDS (double buffer). All
  // loads are ordinary loads, so the compiler's waits cover exactly the data
  // each step uses. Iteration ch: A(ch+1) registers -> LDS; load A(ch+2) and
  // X(ch+3); multiply chunk ch; barrier.
  bf16x8 xr[4][4];
  u32x4 ar[kAJ];
  load_a(0, ar);
  load_x(0, xr[0]);
  if (1 < nchunks) load_x(1, xr[1]);
  if (2 < nchunks) load_x(2, xr[2]);
  store_a(ar, 0);
  if (1 < nchunks) load_a(1, ar);
  __syncthreads();
  auto step = [&](int ch, auto ring) {
    constexpr int R = decltype(ring)::value;  // ch % 4
    if (ch + 1 < nchunks) store_a(ar, (R + 1) & 1);
    if (ch + 2 < nchunks) load_a(ch + 2, ar);
    if (ch + 3 < nchunks) load_x(ch + 3, xr[(R + 3) & 3]);
    const __bf16* ab = abuf + (R & 1) * ABUF;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 af =
            *reinterpret_cast<const bf16x8*>(ab + ((2 * ks + hi) * NA_PAD + 32 * mt + l32) * 8);
        acc[mt] = mfma32x32x16(af, xr[R][ks], acc[mt]);
      }
    }
    __syncthreads();
  };
  for (int ch = 0; ch < nchunks; ch += 4) {
    step(ch, std::integral_constant<int, 0>{});
    if (ch + 1 < nchunks) step(ch + 1, std::integral_constant<int, 1>{});
    if (ch + 2 < nchunks) step(ch + 2, std::integral_constant<int, 2>{});
    if (ch + 3 < nchunks) step(ch + 3, std::integral_constant<int, 3>{});
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

  // g^2 z^2 = sum over tile pairs of p_mt . (G[mt][kt] p_kt), kt >= mt, the
  // off-diagonal pairs twice (G is symmetric). Each pair's G operands (16
  // floats per lane, stored in operand order) are loaded one pair ahead.
  const float4* gl = reinterpret_cast<const float4*>(gsw) + 4 * lane;
  float4 gn[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) gn[v] = gl[v];
  float gsq = 0.f;
  int p = 0;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    float part = 0.f;
#pragma unroll
    for (int kt = mt; kt < MT; ++kt, ++p) {
      float gc[16];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        gc[4 * v] = gn[v].x;
        gc[4 * v + 1] = gn[v].y;
        gc[4 * v + 2] = gn[v].z;
        gc[4 * v + 3] = gn[v].w;
      }
      if (p + 1 < gram_pairs(MT)) {
#pragma unroll
        for (int v = 0; v < 4; ++v) gn[v] = gl[256 * (p + 1) + v];
      }
      f32x16 y = {};
#pragma unroll
      for (int r = 0; r < 16; ++r)
        y = __builtin_amdgcn_mfma_f32_32x32x2f32(gc[r], acc[kt][r], y, 0, 0, 0);
      float d = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) d = fmaf(y[r], acc[mt][r], d);
      part += kt == mt ? d : 2.f * d;
    }
    gsq += part;
  }
  gsq += __shfl_xor(gsq, 32);
  if (hi == 0 && tok_ok) gout[tok] = sqrtf(fmaxf(gsq, 0.f)) / z;
}

// ------------------------------------------------------- line sum partials --
// Partials per (zone, chunk of kLC channels): [0] sum x^2, [1..3] sum over the
// lines along t, h, w of (line sum)^2 / line length, in fp64 (for bf16 inputs
// the sums and squares are exact; the division by the length is a multiply by
// its rounded reciprocal). The zone is held in LDS as t-slices of 16 x 16
// tokens x kLC channels: w- and h-lines are complete inside a slice, t-lines
// accumulate in registers across slices. bf16 features: the whole zone (up to
// 4 slices, 64 KB) is requested at once with direct global->LDS loads (pad
// tokens read as zero through the buffer bounds), so one memory latency is
// paid per workgroup; the one-channel fp32 field is staged a slice at a time.
// Each thread owns fixed lines and the workgroup reduction has a fixed order
// (deterministic).
constexpr int kLC = 32;   // channels per workgroup
constexpr int kLT = 512;  // threads per workgroup
constexpr int kTI = 256 * kLC / kLT;  // t-line items per thread

template <typename T>
__global__ __launch_bounds__(kLT) void line_kernel(Lay L, const T* __restrict__ X, int C,
                                                   double* __restrict__ part) {
  constexpr bool kDirect = sizeof(T) == 2;  // bf16: whole zone by direct loads
  constexpr int kSlice = 16 * 16 * kLC;     // elements of one t-slice: [h][w][c]
  __shared__ __align__(16) T xs[(kDirect ? 4 : 1) * kSlice];
  __shared__ double red[4][kLT / 64];
  const int z = blockIdx.x, chunk = blockIdx.y, nchunks = gridDim.y, tid = threadIdx.x;
  const int zzt = z / (L.gzh * L.gzw), zzh = (z / L.gzw) % L.gzh, zzw = z % L.gzw;
  const int t0 = zzt * L.zt, h0 = zzh * L.zh, w0 = zzw * L.zw;
  const int vt = imax(0, imin(L.zt, L.T - t0));
  const int vh = imax(0, imin(L.zh, L.H - h0));
  const int vw = imax(0, imin(L.zw, L.W - w0));
  const int c0 = chunk * kLC;
  constexpr int EPC = 16 / sizeof(T);   // elements per 16-byte load
  constexpr int NSEG = kLC / EPC;       // 16-byte segments per token
  const bool vec = (C % EPC) == 0;
  const double inv_vw = vw ? 1.0 / vw : 0.0, inv_vh = vh ? 1.0 / vh : 0.0;
  const double inv_vt = vt ? 1.0 / vt : 0.0;
  double q = 0.0, rh = 0.0, rw = 0.0;
  double tacc[kTI];  // t-line sums of items tid + kLT j: channel item % 32, token item / 32
#pragma unroll
  for (int j = 0; j < kTI; ++j) tacc[j] = 0.0;
  if constexpr (kDirect) {
    // LDS slot s (16 bytes) = token s / NSEG of the zone ([t][h][w]), segment
    // s % NSEG; wave u % 8 loads slots 64 u .. 64 u + 63. Offsets are relative
    // to the zone's first token (the host requires zt H W C 2 < 2^31); pad and
    // out-of-grid tokens take an offset past the buffer and read zero.
    constexpr uint32_t kPadOff = 0x7ffffff0u;  // >= the buffer size below: reads zero
    const size_t base = (((size_t)t0 * L.H + h0) * L.W + w0) * (size_t)C + c0;
    const size_t left = ((size_t)L.N * C - base) * sizeof(T);  // bytes from base to X's end
    const i32x4 rs = make_buffer_rsrc(X + base, (uint32_t)(left < kPadOff ? left : kPadOff));
    const int w = tid >> 6, lane = tid & 63;
    const int units = vt * 256 * NSEG / 64;  // 16 per slice
    for (int u = w; u < units; u += kLT / 64) {
      const int sl = 64 * u + lane, k = sl / NSEG, sg = sl % NSEG;
      const int tt = k >> 8, th = (k >> 4) & 15, tw = k & 15;
      const bool real = th < vh && tw < vw;
      const int off = real ? (int)((((size_t)tt * L.H + th) * L.W + tw) * (size_t)C * 2 + 16 * sg)
                           : (int)kPadOff;
      dma16_manual(rs, lds_addr_of(xs + (size_t)64 * u * EPC), off, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
  }
  for (int tt = 0; tt < vt; ++tt) {
    const T* xsl = xs + (kDirect ? tt * kSlice : 0);
    if constexpr (!kDirect) {
      __syncthreads();
      // stage the slice: token k = 16 th + tw, segment sg
      for (int e = tid; e < 256 * NSEG; e += kLT) {
        const int k = e / NSEG, sg = e % NSEG;
        const int th = k >> 4, tw = k & 15;
        T* dst = xs + k * kLC + sg * EPC;
        const int cc = c0 + sg * EPC;
        if (th < vh && tw < vw) {
          const long long n = ((long long)(t0 + tt) * L.H + (h0 + th)) * L.W + (w0 + tw);
          if (vec && cc + EPC <= C) {
            *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(X + n * C + cc);
          } else {
            for (int qq = 0; qq < EPC; ++qq) dst[qq] = cc + qq < C ? X[n * C + cc + qq] : (T)0.f;
          }
        } else {
          for (int qq = 0; qq < EPC; ++qq) dst[qq] = (T)0.f;
        }
      }
    }
    if constexpr (!kDirect) __syncthreads();
    // w-lines (th, c) and h-lines (tw, c) of this slice, one of each per thread
    {
      const int item = tid, c = item & 31, l = item >> 5;
      double sw = 0.0, sh = 0.0;
      for (int u = 0; u < 16; ++u) {
        const double xw = (double)(float)xsl[(l * 16 + u) * kLC + c];  // (th = l, tw = u)
        const double xh = (double)(float)xsl[(u * 16 + l) * kLC + c];  // (th = u, tw = l)
        sw += xw;
        q += xw * xw;
        sh += xh;
      }
      rw += l < vh ? sw * sw * inv_vw : 0.0;
      rh += l < vw ? sh * sh * inv_vh : 0.0;
    }
#pragma unroll
    for (int j = 0; j < kTI; ++j) {
      const int item = tid + kLT * j;
      tacc[j] += (double)(float)xsl[(item >> 5) * kLC + (item & 31)];
    }
  }
  double rt = 0.0;
#pragma unroll
  for (int j = 0; j < kTI; ++j) rt += tacc[j] * tacc[j] * inv_vt;
  // workgroup reduction in a fixed order (deterministic)
  double vals[4] = {q, rt, rh, rw};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    double v = vals[k];
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if ((tid & 63) == 0) red[k][tid >> 6] = v;
  }
  __syncthreads();
  if (tid < 4) {
    double sres = 0.0;
    for (int v = 0; v < kLT / 64; ++v) sres += red[tid][v];
    part[((size_t)z * nchunks + chunk) * 4 + tid] = sres;
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

// Workspace: g [N] f32 | gram [pad^2] f32 (upper tile pairs use less) | xpart [nZ][chunks][4] | gpart [nZ][4] | scratch [7 nZ]
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
    gram_kernel<<<gram_pairs(pad / 32), 64, 0, st>>>(A, n_audio, pad / 32, C, gram);
    const unsigned grid = (unsigned)((L.N + kTok - 1) / kTok);  // C % 64 == 0 (checked)
    const float isc = 1.0f / sqrtf((float)C);
    switch (pad / 32) {
#define BSA_A2V(MT) \
  case MT: a2v_kernel<MT><<<grid, 64 * kA2vWaves, 0, st>>>(X, C, L.N, A, n_audio, gram, isc, g); break;
      BSA_A2V(1) BSA_A2V(2) BSA_A2V(3) BSA_A2V(4) BSA_A2V(5) BSA_A2V(6) BSA_A2V(7) BSA_A2V(8)
#undef BSA_A2V
      default: return hipErrorInvalidValue;
    }
    line_kernel<float><<<dim3(L.nZ, 1), kLT, 0, st>>>(L, g, 1, gpart);
  }
  line_kernel<__bf16><<<dim3(L.nZ, chunks), kLT, 0, st>>>(L, X, C, xpart);
  decide_kernel<<<1, 256, 0, st>>>(L, C, chunks, xpart, gpart, use_audio ? 1 : 0, zone_shape,
                                   zone_stats, scratch);
  return hipGetLastError();
}

}  // namespace bsa

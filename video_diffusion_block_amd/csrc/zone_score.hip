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
//                  the upper tile pairs, each split into three bf16 pieces
//                  (hi + mid + lo: 24 significant bits, as many as fp32) in
//                  the A2V kernel's operand order.
//  a2v_kernel      per 256 tokens: logits^T = A X^T on bf16 MFMA (exact products,
//                  fp32 sums), softmax in fp32 registers (lane-local rows), then
//                  g^2 = p^T G p as Y = G P^T over the upper tile pairs of the
//                  symmetric G and a lane-local dot with P. Y is formed on
//                  bf16 MFMA from three-piece splits of G and P (the six
//                  products whose pieces carry the top 24 bits; exact
//                  products, fp32 sums), which matches an fp32 product in
//                  6/16 of its matrix-unit time. Writes g [N] fp32.
//  line_kernel     per (zone, 32-channel chunk): the zone is streamed through
//                  LDS one t-slice at a time; sum x^2 and the squared line sums
//                  along t, h, w in fp64 (bf16 inputs make these sums exact), so
//                  V_a = (sum x^2 - sum_lines S^2/len) / (C n_z). The chunk-0
//                  workgroup of each zone also sums the one-channel field g.
//  decide_kernel   one workgroup: sum the chunk partials in a fixed order,
//                  the means, r, the costs and the tie rule; writes the shape
//                  ids.
#include <math.h>

#include <type_traits>

#include "attn_common.hpp"
#include "kernels.hpp"

namespace bsa {
namespace {

constexpr double kTieRel = 1e-6;

// ------------------------------------------------------------- Gram matrix --
// x = hi + mid + lo with each piece the bf16 rounding of what the previous
// ones leave (the two subtractions are exact), so the pieces hold the top 24
// significant bits of x; the residual is below 2^-24 |x|.
// Element r of a 16-value lane row goes to element r % 8 of piece[k][r / 8].
__device__ inline void split3(float x, bf16x8 (&piece)[3][2], int r) {
  const __bf16 hi = (__bf16)x;
  const float r1 = x - (float)hi;
  const __bf16 mid = (__bf16)r1;
  piece[0][r >> 3][r & 7] = hi;
  piece[1][r >> 3][r & 7] = mid;
  piece[2][r >> 3][r & 7] = (__bf16)(r1 - (float)mid);
}

// One workgroup of kGramWaves wavefronts per tile pair (mt, kt), kt >= mt, of
// G = A A^T on bf16 MFMA (the products of bf16 values are exact and accumulate
// in fp32; rows past Na read as zero). Wavefront u sums the 64-channel chunks
// u, u + kGramWaves, ...; the partial tiles are added in wavefront order (a
// fixed order: deterministic). The tile is stored split into three bf16
// pieces, in the operand order of the A2V kernel's phase 2: lane
// l = 32 hi + l32 of pair p owns 16 consecutive values of each piece, value
// r = G[32 mt + l32][32 kt + 8 (r / 4) + 4 hi + r % 4] (values 8s .. 8s + 7
// are its A operand of k-step s). The MFMA result of rows kt x columns mt
// has exactly that lane layout (G is symmetric, and G[i][j], G[j][i] are the
// same products summed in the same order).
// Layout of the output: [pair][piece: hi, mid, lo][lane][16] bf16.
constexpr int kGramWaves = 4;
__host__ __device__ constexpr int gram_pairs(int mt_count) { return mt_count * (mt_count + 1) / 2; }

__global__ __launch_bounds__(64 * kGramWaves) void gram_kernel(const __bf16* A, int Na,
                                                               int mt_count, int C, __bf16* gsw) {
  __shared__ f32x16 red[kGramWaves - 1][64];
  const int p = blockIdx.x, lane = threadIdx.x & 63;
  const int u = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int mt = 0, rem = p;
  while (rem >= mt_count - mt) rem -= mt_count - mt++;
  const int kt = mt + rem;
  const int l32 = lane & 31, hi = lane >> 5;
  const int ra = 32 * kt + l32, rb = 32 * mt + l32;
  const __bf16* pa = A + (size_t)ra * C + 8 * hi;
  const __bf16* pb = A + (size_t)rb * C + 8 * hi;
  f32x16 acc = {};
  const bf16x8 zero = {};
  for (int c = 64 * u; c < C; c += 64 * kGramWaves) {
    bf16x8 a[4], b[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {  // C is a multiple of 64
      a[s] = ra < Na ? *reinterpret_cast<const bf16x8*>(pa + c + 16 * s) : zero;
      b[s] = rb < Na ? *reinterpret_cast<const bf16x8*>(pb + c + 16 * s) : zero;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma32x32x16(a[s], b[s], acc);
  }
  if (u > 0) red[u - 1][lane] = acc;
  __syncthreads();
  if (u != 0) return;
#pragma unroll
  for (int v = 0; v < kGramWaves - 1; ++v) acc += red[v][lane];
  bf16x8 pc[3][2];
#pragma unroll
  for (int r = 0; r < 16; ++r) split3(acc[r], pc, r);
  bf16x8* out = reinterpret_cast<bf16x8*>(gsw) + (size_t)p * 3 * 128 + 2 * lane;
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    out[128 * k] = pc[k][0];
    out[128 * k + 1] = pc[k][1];
  }
}

// --------------------------------------------------------------- A2V norm --
// 8 wavefronts x 32 tokens per workgroup. Phase 1, logits^T = A X^T on bf16
// MFMA over 64-channel chunks, every operand through LDS by hand-issued direct
// global->LDS loads (the kernel places its own waits, so no load waits for
// more than the data the next step uses): A, shared by the wavefronts,
// double-buffered and laid out piece-major ([8-channel piece][audio row], rows
// past Na read as zero through the buffer bounds) so the fragment reads are
// conflict free; X, private to each wavefront, in a ring of three chunks
// (each token row read once, in whole 128-byte pieces; pieces swizzled by
// token so the fragment reads are conflict free; rows past N read as zero).
// Phase 2: softmax in fp32 registers, then g^2 z^2 = p^T G p over the tile
// pairs kt >= mt of the symmetric G (off-diagonal pairs counted twice), the
// pairs' G pieces (the Gram kernel's three-piece split, in operand order)
// staged in the freed operand buffers once per workgroup and read from LDS.
// Index of the stored Gram tile pair (mt, kt), kt >= mt (row-major upper
// triangle of an mtc x mtc tile grid), and the end of a round of whole rows
// kt0 .. of the phase-2 loop order that holds at most cap pairs.
__host__ __device__ constexpr int gpair_of(int mtc, int mt, int kt) {
  return mt * mtc - mt * (mt - 1) / 2 + (kt - mt);
}
__host__ __device__ constexpr int stage_end(int mtc, int kt0, int cap) {
  int kt = kt0, n = 0;
  while (kt < mtc && n + kt + 1 <= cap) n += ++kt;
  return kt;
}
constexpr int kA2vWaves = 8;
constexpr int kTok = 32 * kA2vWaves;  // tokens per workgroup
constexpr int kCh = 64;               // channels per chunk
constexpr int kXRing = 3;             // X chunks per wavefront in LDS

template <int MT>
__global__ __launch_bounds__(64 * kA2vWaves) void a2v_kernel(const __bf16* X, int C, long long N,
                                                             const __bf16* A, int Na,
                                                             const __bf16* gsw, float inv_sqrt_c,
                                                             float* gout) {
  constexpr int NA_PAD = 32 * MT;
  constexpr int SLOTS = 8 * NA_PAD;  // 16-byte slots per A chunk: 4 MT wave-loads
  constexpr int ABUF = SLOTS * 8;    // bf16 elements per A buffer
  constexpr int kAL = (4 * MT + kA2vWaves - 1) / kA2vWaves;  // A wave-loads per wave, at most
  // one LDS array: phase 1's A [2][piece][row][8] and X [ring][wave][token][piece][8];
  // phase 2's staged G pieces
  constexpr int kXW = 32 * kCh;  // bf16 elements of one wavefront's X chunk
  constexpr int kSmem = (2 * ABUF + kXRing * kA2vWaves * kXW) * 2;
  __shared__ __align__(16) unsigned char smem[kSmem];
  __bf16* const abuf = reinterpret_cast<__bf16*>(smem);
  __bf16* const xbuf = abuf + 2 * ABUF;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const long long n0 = (long long)blockIdx.x * kTok + 32 * w;  // this wave's first token
  const long long tok = n0 + l32;
  const bool tok_ok = tok < N;
  const int nchunks = C / kCh;
  constexpr int kPadOff = 0x7ffffff0;  // an offset past every buffer below: reads zero

  // A chunk ch into buffer bf: wave-load L = kA2vWaves m + w (L < 4 MT) fills
  // slots 64 L + lane; slot s = piece * NA_PAD + row takes A[row][64 ch +
  // 8 piece .. +8] (Na C 2 <= 4 MiB: offsets fit in 32 bits).
  const i32x4 ars = make_buffer_rsrc(A, (uint32_t)Na * C * 2);
  auto dma_a = [&](int ch, int bf) {
#pragma unroll
    for (int m = 0; m < kAL; ++m) {
      const int L = kA2vWaves * m + w;
      if (L < 4 * MT) {
        const int sl = 64 * L + lane;
        const int piece = sl / NA_PAD, r = sl - piece * NA_PAD;
        const int off = r < Na ? (r * C + kCh * ch + 8 * piece) * 2 : kPadOff;
        dma16_manual(ars, lds_addr_of(abuf + bf * ABUF + 64 * L * 8), off, 0);
      }
    }
  };
  // X chunk ch into ring slot rs: wave-load m fills this wave's slots
  // 64 m + lane: token n = slot / 8 (of the wave's 32), stored piece slot % 8
  // holds logical piece (slot % 8) ^ (n % 8), channels 64 ch + 8 piece .. +8.
  // The buffer covers the wave's rows that exist (32 C 2 <= 512 KiB).
  const long long xrows = N - n0 < 0 ? 0 : (N - n0 < 32 ? N - n0 : 32);
  const i32x4 xrs = make_buffer_rsrc(X + (n0 < N ? n0 : 0) * C, (uint32_t)(xrows * C * 2));
  auto dma_x = [&](int ch, int rs) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int n = 8 * m + (lane >> 3), q = (lane & 7) ^ (n & 7);
      dma16_manual(xrs, lds_addr_of(xbuf + (rs * kA2vWaves + w) * kXW + 64 * m * 8),
                   (n * C + kCh * ch + 8 * q) * 2, 0);
    }
  };

  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;

  // Pipeline: A one chunk ahead, X two ahead. Step ch: wait for A(ch) and
  // X(ch) (the only loads issued after A(ch) are X(ch+1)'s four), barrier
  // (A(ch) complete for every wave; every wave is done with the other A
  // buffer), request A(ch+1) and X(ch+2) (into the ring slot this wave read
  // in step ch-1), multiply chunk ch.
  dma_a(0, 0);
  dma_x(0, 0);
  if (1 < nchunks) dma_x(1, 1);
  auto step = [&](int ch, auto ring) {
    constexpr int R = decltype(ring)::value;  // ch % 3
    if (ch + 1 < nchunks) __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
    else __builtin_amdgcn_s_waitcnt(0x0F70);                   // vmcnt(0)
    __syncthreads();
    if (ch + 1 < nchunks) dma_a(ch + 1, (ch + 1) & 1);
    if (ch + 2 < nchunks) dma_x(ch + 2, (R + 2) % kXRing);
    const __bf16* ab = abuf + (ch & 1) * ABUF;
    const __bf16* xb = xbuf + (R * kA2vWaves + w) * kXW;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 bx =
          *reinterpret_cast<const bf16x8*>(xb + (l32 * 8 + ((2 * ks + hi) ^ (l32 & 7))) * 8);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 af =
            *reinterpret_cast<const bf16x8*>(ab + ((2 * ks + hi) * NA_PAD + 32 * mt + l32) * 8);
        acc[mt] = mfma32x32x16(af, bx, acc[mt]);
      }
    }
  };
  for (int ch = 0; ch < nchunks; ch += 3) {
    step(ch, std::integral_constant<int, 0>{});
    if (ch + 1 < nchunks) step(ch + 1, std::integral_constant<int, 1>{});
    if (ch + 2 < nchunks) step(ch + 2, std::integral_constant<int, 2>{});
  }

  constexpr int kPairBytes = 3 * 2 * 64 * 16;
  constexpr int kCap = kSmem / kPairBytes;  // pairs per round
  constexpr int kE1 = stage_end(MT, 0, kCap), kE2 = stage_end(MT, kE1, kCap);
  static_assert(kE2 == MT, "the Gram pieces must fit in two rounds");
  const i32x4 grs = make_buffer_rsrc(gsw, (uint32_t)gram_pairs(MT) * kPairBytes);
  // stage the pairs of rows kt0 .. kt1-1: wave-load L = q * 6 + 2 piece + s
  auto stage_dma = [&](int kt0, int kt1) {
    const int np = (kt1 * (kt1 + 1) - kt0 * (kt0 + 1)) / 2;
    for (int L = w; L < 6 * np; L += kA2vWaves) {  // (wave-uniform)
      const int q = L / 6, k = (L % 6) >> 1, sb = L & 1;
      int kt = kt0, first = 0;  // row of stage pair q and its first pair
      while (first + kt + 1 <= q) first += ++kt;
      const int pr = gpair_of(MT, q - first, kt);
      dma16_manual(grs, lds_addr_of(smem + (size_t)L * 64 * 16),
                   (384 * pr + 128 * k + 2 * lane + sb) * 16, 0);
    }
  };
  // Phase 2's first round of G pieces replaces the operand buffers: requested
  // once every wavefront is past its phase-1 reads, landing during the softmax.
  __syncthreads();
  stage_dma(0, kE1);

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
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's G loads have landed
  __syncthreads();                      // and every wave's

  // g^2 z^2 = sum over tile pairs of p_mt . (G[mt][kt] p_kt), kt >= mt, the
  // off-diagonal pairs twice (G is symmetric). Y = G[mt][kt] P_kt on bf16
  // MFMA from the three-piece splits of G (stored by the Gram kernel) and of
  // P_kt (split once per kt): the six products hi.hi, hi.mid, mid.hi, hi.lo,
  // mid.mid, lo.hi, smallest first. Lane-local element r of acc[kt] is P at
  // audio 32 kt + 8 (r / 4) + 4 hi + r % 4, the k index the stored G pieces
  // use, so elements 8s .. 8s + 7 are the B operand of k-step s as they lie.
  // The G pieces are staged in LDS once per workgroup (every wavefront needs
  // every pair), in the loop order (kt, then mt <= kt), in at most two rounds
  // of whole kt rows that fit the operand buffers: slot ((q 3 + piece) 2 + s)
  // 64 + lane holds 16 bytes (lanes contiguous: conflict-free reads).
  float gsq = 0.f;
  auto stage_run = [&](auto kt0c, auto kt1c) {
    constexpr int KT0 = decltype(kt0c)::value, KT1 = decltype(kt1c)::value;
#pragma unroll
    for (int kt = KT0; kt < KT1; ++kt) {
      bf16x8 pp[3][2];
#pragma unroll
      for (int r = 0; r < 16; ++r) split3(acc[kt][r], pp, r);
#pragma unroll
      for (int mt = 0; mt <= kt; ++mt) {
        const int q = (kt * (kt + 1) - KT0 * (KT0 + 1)) / 2 + mt;
        bf16x8 gc[3][2];
#pragma unroll
        for (int k = 0; k < 3; ++k)
#pragma unroll
          for (int sb = 0; sb < 2; ++sb)
            gc[k][sb] = *reinterpret_cast<const bf16x8*>(
                smem + ((size_t)((q * 3 + k) * 2 + sb) * 64 + lane) * 16);
        f32x16 y = {};
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          y = mfma32x32x16(gc[2][sb], pp[0][sb], y);  // lo . hi
          y = mfma32x32x16(gc[1][sb], pp[1][sb], y);  // mid . mid
          y = mfma32x32x16(gc[0][sb], pp[2][sb], y);  // hi . lo
        }
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          y = mfma32x32x16(gc[1][sb], pp[0][sb], y);  // mid . hi
          y = mfma32x32x16(gc[0][sb], pp[1][sb], y);  // hi . mid
        }
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) y = mfma32x32x16(gc[0][sb], pp[0][sb], y);  // hi . hi
        float d = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) d = fmaf(y[r], acc[mt][r], d);
        gsq += kt == mt ? d : 2.f * d;
      }
    }
  };
  stage_run(std::integral_constant<int, 0>{}, std::integral_constant<int, kE1>{});
  if constexpr (kE1 < MT) {
    __syncthreads();  // every wavefront is done with the first round
    stage_dma(kE1, MT);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    stage_run(std::integral_constant<int, kE1>{}, std::integral_constant<int, MT>{});
  }
  gsq += __shfl_xor(gsq, 32);
  if (hi == 0 && tok_ok) gout[tok] = sqrtf(fmaxf(gsq, 0.f)) / z;
}

// ------------------------------------------------------- line sum partials --
// Partials per (zone, chunk of kLC = 32 channels) of the bf16 features: [0]
// sum x^2, [1..3] sum over the lines along t, h, w of (line sum)^2 / line
// length, in fp64 (bf16 inputs make the sums and squares exact; the division
// by the length is a multiply by its rounded reciprocal). The zone's t-slices
// (16 x 16 tokens x 32 channels, 16 KB each) stream through two LDS buffers
// with direct global->LDS loads (pad tokens read as zero through the buffer
// bounds), one slice ahead of the one being summed; 37 KB of LDS lets four
// workgroups share a CU. Two walks read a
// slice: thread (h, channel pair) walks its two w-lines (line sums, sum of
// squares, and the t-line sums of its 16 tokens, kept in registers across
// slices); thread (w, channel pair) walks its two h-lines. Token (h, w) sits
// at LDS position 16 h + (w ^ (h & 3)) (64 bytes each), so the four h (or w)
// values a wavefront reads at once fall in different bank groups: both walks
// are conflict free. Pad tokens are zero, so their lines add nothing and no
// masks are needed. The chunk-0 workgroup of a zone also takes the one-channel
// fp32 field g when one is given (its sums of fp32 values are exact in fp64
// too). Every reduction has a fixed order (deterministic).
constexpr int kLC = 32;   // channels per workgroup
constexpr int kLT = 256;  // threads per workgroup

__device__ inline double wave_sum_f64(double x) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__global__ __launch_bounds__(kLT) void line_kernel(Lay L, const __bf16* __restrict__ X, int C,
                                                   const float* __restrict__ g,
                                                   double* __restrict__ xpart,
                                                   double* __restrict__ gpart) {
  __shared__ __align__(16) uint32_t xs[2][16 * 16 * kLC / 2];  // [buffer][position][16 dwords]
  __shared__ float gs[4][256];
  __shared__ double red[4][kLT / 64];
  const int z = blockIdx.x, chunk = blockIdx.y, nchunks = gridDim.y, tid = threadIdx.x;
  const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int zzt = z / (L.gzh * L.gzw), zzh = (z / L.gzw) % L.gzh, zzw = z % L.gzw;
  const int t0 = zzt * L.zt, h0 = zzh * L.zh, w0 = zzw * L.zw;
  const int vt = imax(0, imin(L.zt, L.T - t0));
  const int vh = imax(0, imin(L.zh, L.H - h0));
  const int vw = imax(0, imin(L.zw, L.W - w0));
  const double inv_vw = vw ? 1.0 / vw : 0.0, inv_vh = vh ? 1.0 / vh : 0.0;
  const double inv_vt = vt ? 1.0 / vt : 0.0;

  // Loads of slice tt into buffer buf: load m (0..3) of wave wv fills 16-byte
  // slots (4 m + wv) * 64 + lane: position slot / 4, channels 8 (slot % 4) ..
  // +8. Offsets are relative to the zone's first token (the host requires
  // zt H W C 2 < 2^31); pad and out-of-grid tokens take an offset past the
  // buffer and read zero.
  constexpr uint32_t kPadOff = 0x7ffffff0u;  // >= the buffer size below: reads zero
  const size_t base = (((size_t)t0 * L.H + h0) * L.W + w0) * (size_t)C + (size_t)chunk * kLC;
  const size_t left = ((size_t)L.N * C - base) * 2;  // bytes from base to X's end
  const i32x4 rs = make_buffer_rsrc(X + base, (uint32_t)(left < kPadOff ? left : kPadOff));
  auto issue = [&](int tt, int buf) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int sl = (4 * m + wv) * 64 + lane;
      const int pos = sl >> 2, th = pos >> 4, tw = (pos & 15) ^ (th & 3);
      const bool real = th < vh && tw < vw;
      const int off = real ? (int)((((size_t)tt * L.H + th) * L.W + tw) * (size_t)C * 2 +
                                   16 * (sl & 3))
                           : (int)kPadOff;
      dma16_manual(rs, lds_addr_of(&xs[buf][(4 * m + wv) * 256]), off, 0);
    }
  };
  issue(0, 0);
  if (vt > 1) issue(1, 1);
  // a = h of the w-walk and w of the h-walk; cp = channel pair (dword) of the token
  const int a = 4 * wv + (lane >> 4), cp = lane & 15;
  double tacc[16][2];
#pragma unroll
  for (int u = 0; u < 16; ++u) tacc[u][0] = tacc[u][1] = 0.0;
  double q = 0.0, rw = 0.0, rh = 0.0;
  for (int tt = 0; tt < vt; ++tt) {
    // this wave's loads of slices 0..tt have landed (4 loads per slice), then
    // every wave's
    // this wave's loads of slice tt have landed (the next slice's four may
    // be in flight), then every wave's
    if (tt + 1 < vt) __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
    else __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0)
    __syncthreads();
    const uint32_t* sl = xs[tt & 1];
    double sw0 = 0.0, sw1 = 0.0, sh0 = 0.0, sh1 = 0.0;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const uint32_t vw_ = sl[(16 * a + (u ^ (a & 3))) * 16 + cp];  // token (h = a, w = u)
      const uint32_t vh_ = sl[(16 * u + (a ^ (u & 3))) * 16 + cp];  // token (h = u, w = a)
      const double x0 = (double)__uint_as_float(vw_ << 16);
      const double x1 = (double)__uint_as_float(vw_ & 0xffff0000u);
      sw0 += x0;
      sw1 += x1;
      q = fma(x0, x0, q);
      q = fma(x1, x1, q);
      tacc[u][0] += x0;
      tacc[u][1] += x1;
      sh0 += (double)__uint_as_float(vh_ << 16);
      sh1 += (double)__uint_as_float(vh_ & 0xffff0000u);
    }
    rw += (sw0 * sw0 + sw1 * sw1) * inv_vw;
    rh += (sh0 * sh0 + sh1 * sh1) * inv_vh;
    if (tt + 2 < vt) {
      __syncthreads();  // every wave is done with this buffer
      issue(tt + 2, tt & 1);
    }
  }
  double rt = 0.0;
#pragma unroll
  for (int u = 0; u < 16; ++u) rt += (tacc[u][0] * tacc[u][0] + tacc[u][1] * tacc[u][1]) * inv_vt;

  // workgroup sums in a fixed order: lanes (butterfly), then waves in order
  auto block_sum4 = [&](const double (&v)[4], double* out) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const double x = wave_sum_f64(v[k]);
      if (lane == 0) red[k][wv] = x;
    }
    __syncthreads();
    if (tid < 4) {
      double sres = 0.0;
      for (int u = 0; u < kLT / 64; ++u) sres += red[tid][u];
      out[tid] = sres;
    }
  };
  const double vals[4] = {q, rt, rh, rw};
  block_sum4(vals, xpart + ((size_t)z * nchunks + chunk) * 4);

  if (g == nullptr || chunk != 0) return;
  // the field g of the zone: thread (h, w) = (tid / 16, tid % 16) stages its
  // t-line and sums it; threads 0..63 take the w-lines (t, h), 64..127 the
  // h-lines (t, w)
  const int gh_ = tid >> 4, gw_ = tid & 15;
  for (int tt = 0; tt < 4; ++tt) {
    float v = 0.f;
    if (tt < vt && gh_ < vh && gw_ < vw)
      v = g[((long long)(t0 + tt) * L.H + (h0 + gh_)) * L.W + (w0 + gw_)];
    gs[tt][tid] = v;
  }
  __syncthreads();  // (also: the X sums have read red)
  double gq = 0.0, gst = 0.0, gsh = 0.0, gsw = 0.0;
  {
    double st = 0.0;
    for (int tt = 0; tt < vt; ++tt) {
      const double x = gs[tt][tid];
      st += x;
      gq = fma(x, x, gq);
    }
    gst = st * st * inv_vt;
  }
  if (tid < 64) {
    const int tt = tid >> 4, hh = tid & 15;
    if (tt < vt) {
      double sres = 0.0;
      for (int ww = 0; ww < 16; ++ww) sres += gs[tt][16 * hh + ww];
      gsw = sres * sres * inv_vw;
    }
  } else if (tid < 128) {
    const int tt = (tid - 64) >> 4, ww = tid & 15;
    if (tt < vt) {
      double sres = 0.0;
      for (int hh = 0; hh < 16; ++hh) sres += gs[tt][16 * hh + ww];
      gsh = sres * sres * inv_vh;
    }
  }
  const double gvals[4] = {gq, gst, gsh, gsw};
  block_sum4(gvals, gpart + 4 * (size_t)z);
}

// ------------------------------------------------------------------ decide --
// One workgroup. Phase 1: thread (zone, component) sums the zone's chunk
// partials of that component in chunk order. Phase 2: per zone V_a, G_a and
// the size; the means over non-empty (zone, axis) pairs by a fixed-order tree.
// Phase 3: per zone r_a, the costs and the tie rule. Deterministic.
constexpr int kDecideThreads = 1024;
__global__ __launch_bounds__(kDecideThreads) void decide_kernel(
    Lay L, int C, int nchunks, const double* xpart, const double* gpart, int use_audio,
    int32_t* zone_shape, double* zone_stats, double* scratch) {
  // scratch: V [nZ][3], G [nZ][3], nz [nZ], chunk sums [nZ][4]
  double* V = scratch;
  double* G = scratch + 3 * L.nZ;
  double* NZ = scratch + 6 * L.nZ;
  double* S = scratch + 7 * L.nZ;
  __shared__ double sv[kDecideThreads], sg[kDecideThreads];
  __shared__ int scount[kDecideThreads];
  const int tid = threadIdx.x;
  for (int e = tid; e < 4 * L.nZ; e += kDecideThreads) {
    const double* p = xpart + (size_t)(e >> 2) * nchunks * 4 + (e & 3);
    double acc = 0.0;
#pragma unroll 8
    for (int k = 0; k < nchunks; ++k) acc += p[4 * k];
    S[e] = acc;
  }
  __syncthreads();
  double accv = 0.0, accg = 0.0;
  int cnt = 0;
  for (int z = tid; z < L.nZ; z += kDecideThreads) {
    const int zzt = z / (L.gzh * L.gzw), zzh = (z / L.gzw) % L.gzh, zzw = z % L.gzw;
    const int vt = imax(0, imin(L.zt, L.T - zzt * L.zt));
    const int vh = imax(0, imin(L.zh, L.H - zzh * L.zh));
    const int vw = imax(0, imin(L.zw, L.W - zzw * L.zw));
    const double nz = (double)vt * vh * vw;
    NZ[z] = nz;
    const double q = S[4 * z];
    const double r[3] = {S[4 * z + 1], S[4 * z + 2], S[4 * z + 3]};
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
  for (int s = kDecideThreads / 2; s > 0; s >>= 1) {
    if (tid < s) {
      sv[tid] += sv[tid + s];
      sg[tid] += sg[tid + s];
      scount[tid] += scount[tid + s];
    }
    __syncthreads();
  }
  const double vbar = scount[0] ? sv[0] / scount[0] : 0.0;
  const double gbar = scount[0] ? sg[0] / scount[0] : 0.0;
  for (int z = tid; z < L.nZ; z += kDecideThreads) {
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
// three bf16 pieces of 64 lanes x 16 values per upper tile pair
size_t gram_bytes(int mt_count) { return (size_t)gram_pairs(mt_count) * 3 * 64 * 16 * 2; }

}  // namespace

// Workspace: g [N] f32 | gram: pairs x 3 pieces x 2 KB bf16 | xpart [nZ][chunks][4] |
// gpart [nZ][4] | scratch [11 nZ]
size_t zone_score_workspace(const Lay& L, int C, int n_audio) {
  const int pad = 32 * ((n_audio + 31) / 32);
  const int chunks = (C + kLC - 1) / kLC;
  return al256((size_t)L.N * sizeof(float)) + al256(gram_bytes(pad / 32)) +
         al256((size_t)L.nZ * chunks * 4 * sizeof(double)) +
         al256((size_t)L.nZ * 4 * sizeof(double)) + al256((size_t)L.nZ * 11 * sizeof(double));
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
  __bf16* gram = reinterpret_cast<__bf16*>(p);
  p += al256(gram_bytes(pad / 32));
  double* xpart = reinterpret_cast<double*>(p);
  p += al256((size_t)L.nZ * chunks * 4 * sizeof(double));
  double* gpart = reinterpret_cast<double*>(p);
  p += al256((size_t)L.nZ * 4 * sizeof(double));
  double* scratch = reinterpret_cast<double*>(p);

  const __bf16* X = static_cast<const __bf16*>(video);
  const bool use_audio = audio != nullptr && n_audio > 0;
  if (use_audio) {
    const __bf16* A = static_cast<const __bf16*>(audio);
    gram_kernel<<<gram_pairs(pad / 32), 64 * kGramWaves, 0, st>>>(A, n_audio, pad / 32, C, gram);
    const unsigned grid = (unsigned)((L.N + kTok - 1) / kTok);  // C % 64 == 0 (checked)
    const float isc = 1.0f / sqrtf((float)C);
    switch (pad / 32) {
#define BSA_A2V(MT) \
  case MT: a2v_kernel<MT><<<grid, 64 * kA2vWaves, 0, st>>>(X, C, L.N, A, n_audio, gram, isc, g); break;
      BSA_A2V(1) BSA_A2V(2) BSA_A2V(3) BSA_A2V(4) BSA_A2V(5) BSA_A2V(6) BSA_A2V(7) BSA_A2V(8)
#undef BSA_A2V
      default: return hipErrorInvalidValue;
    }
  }
  line_kernel<<<dim3(L.nZ, chunks), kLT, 0, st>>>(L, X, C, use_audio ? g : nullptr, xpart, gpart);
  decide_kernel<<<1, kDecideThreads, 0, st>>>(L, C, chunks, xpart, gpart, use_audio ? 1 : 0, zone_shape,
                                   zone_stats, scratch);
  return hipGetLastError();
}

}  // namespace bsa

// Internal launchers of the HIP kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "layout.hpp"

namespace bsa {

// Gather [heads, N, d] -> [heads, Np, d] (inverse = false) or the reverse.
// Gather (inverse = false) or scatter of up to four tensors. Gather options
// (d in {64, 128}; epc = elements per 16 bytes: 8 bf16 / 4 fp32): tensors
// 0 .. nrope-1 get RMSNorm (weights gamma[t] [d] fp32 or null, eps) and the
// 3-D rotary embedding (base rope_base) before they are stored; the block
// means of tensors 0 .. npool-1 over real slots, of the stored values, go to
// pooled[t] [heads, M, d] fp64 (0 for empty blocks).
hipError_t launch_permute(const Lay& L, const int32_t* zone_shape, int ntensors,
                          const void* const* src, void* const* dst, int heads, int row_bytes,
                          bool inverse, hipStream_t st, int npool = 0,
                          double* const* pooled = nullptr, int epc = 0, int nrope = 0,
                          const float* const* gamma = nullptr, float eps = 0.f,
                          float rope_base = 0.f);




// Per-block facts the attention kernels need inside their loops: bit r of
// mask word r / 32 (r < B) = slot r is real; count = real slots. Stored as two
// 16-byte halves, half h = {word 2h, word 2h + 1, count, x_h}, so that a reader
// of slots 64h .. 64h + 63 gets its words and the count in one load; x_0 is
// the block origin's raster token index on the padded grid and x_1 its shape id.
struct BlockMeta {
  uint32_t half[2][4];
  __host__ __device__ uint32_t mask(int k) const { return half[k >> 1][k & 1]; }
  __host__ __device__ int count() const { return (int)half[0][2]; }
  __host__ __device__ uint32_t origin() const { return half[0][3]; }
  __host__ __device__ int shape() const { return (int)half[1][3]; }
};
hipError_t launch_block_meta(const Lay& L, const int32_t* zone_shape, BlockMeta* meta,
                             hipStream_t st);

// Block means of Q and K over real slots, fp64: [heads, M, d] each.
hipError_t launch_pool(const Lay& L, const BlockMeta* meta, const void* qp, const void* kp,
                       int heads, int d, bool bf16, double* qbar, double* kbar, hipStream_t st);

// Pooled logits l[h,i,j] = qbar_i . kbar_j * scale (fp64), -inf for empty key blocks.
hipError_t launch_pooled_logits(const Lay& L, const BlockMeta* meta, const double* qbar,
                                const double* kbar, int heads, int d, double scale,
                                double* logits, hipStream_t st);

// Hybrid selection per (head, query block) from the pooled logits;
// frames_per_chunk > 0 (a multiple of L.zt) restricts row i to the key blocks
// of its own and earlier frame chunks.
hipError_t launch_select(const Lay& L, const BlockMeta* meta, const double* logits, int heads,
                         int sparsity_1e4, double tau, int32_t* counts, int32_t* idx,
                         hipStream_t st, int frames_per_chunk = 0);

// Attention forward. bf16 + d = 128 + B = 128 takes the MFMA kernel, which
// needs attn_fwd_workspace() bytes (the block table). raster (MFMA kernel
// only): O and lse are written in raster token order, [heads, N, d] and
// [heads, N], instead of the permuted [heads, Np, d] and [heads, Np].
// gather (MFMA kernel, layouts with attn_fwd_gather_ok): Q, K, V are read in
// raster token order, [heads, N, d], and O, lse are written in it.
bool attn_fwd_uses_mfma(const Lay& L, int d, bool bf16);
bool attn_fwd_gather_ok(const Lay& L, int d, bool bf16);
size_t attn_fwd_workspace(const Lay& L, int d, bool bf16);
hipError_t launch_attn_fwd(const Lay& L, const int32_t* zone_shape, const void* qp,
                           const void* kp, const void* vp, const int32_t* counts,
                           const int32_t* idx, int heads, int d, bool bf16, float scale,
                           void* op, float* lse, void* ws, hipStream_t st, bool raster = false,
                           bool gather = false);

// Device address and size of the forward's static scratch array on the
// current device (looked up once per device; no allocation).
hipError_t attn_fwd_static_scratch(void** ptr, size_t* bytes);

// Attention backward. raster (MFMA kernels only: bf16, d = 128, B = 128):
// dQ, dK, dV are written in raster token order, [heads, N, d], instead of
// the permuted [heads, Np, d].
size_t attn_bwd_workspace(const Lay& L, int heads, int d);
hipError_t launch_attn_bwd(const Lay& L, const int32_t* zone_shape, const void* qp,
                           const void* kp, const void* vp, const void* op, const void* dop,
                           const float* lse, const int32_t* counts, const int32_t* idx,
                           int heads, int d, bool bf16, float scale, void* dqp, void* dkp,
                           void* dvp, void* ws, hipStream_t st, bool raster = false);

// A2V cross-attention layer. C[M,N] = sum_k A[m][k] B[n][k] (bf16, K a
// multiple of 8, rows 16-byte aligned), fp32 accumulation, bf16 or fp32 out
// (fp32 optionally added to C).
hipError_t launch_gemm_nt(const __bf16* A, int lda, const __bf16* B, int ldb, int M, int N, int K,
                          void* C, int ldc, bool out_f32, bool accumulate, hipStream_t st);
// bf16 [R, Cc] (row stride lds) -> [Cc, ldo], columns R..ldo-1 zero.
hipError_t launch_transpose(const __bf16* src, int R, int Cc, int lds, __bf16* dst, int ldo,
                            hipStream_t st);
int xattn_na_pad(int n_audio);
// Forward: q [N, H 128], k, v [Na, H 128], o [N, H 128], y [N, C] bf16; lse [H, N].
hipError_t launch_xattn_fwd(int N, int Na, int heads, const __bf16* x, const __bf16* a, int C,
                            const __bf16* wq, const __bf16* wk, const __bf16* wv,
                            const __bf16* wo, __bf16* q, __bf16* k, __bf16* v, __bf16* o,
                            float* lse, __bf16* y, hipStream_t st);

// Backward: gradients of sum(Y * dY) as fp32 (dx [N, C], da [Na, C], dwq,
// dwk, dwv [D, C], dwo [C, D]) from the forward's q, k, v, o, lse.
size_t xattn_bwd_workspace(int N, int Na, int C, int heads);
hipError_t launch_xattn_bwd(int N, int Na, int heads, const __bf16* x, const __bf16* a, int C,
                            const __bf16* wq, const __bf16* wk, const __bf16* wv,
                            const __bf16* wo, const __bf16* q, const __bf16* k, const __bf16* v,
                            const __bf16* o, const float* lse, const __bf16* dy, float* dx,
                            float* da, float* dwq, float* dwk, float* dwv, float* dwo, void* ws,
                            hipStream_t st);

// Zone scoring.
size_t zone_score_workspace(const Lay& L, int C, int n_audio);
hipError_t launch_zone_score(const Lay& L, const void* video, int C, const void* audio,
                             int n_audio, int32_t* zone_shape, double* zone_stats, void* ws,
                             hipStream_t st);

}  // namespace bsa

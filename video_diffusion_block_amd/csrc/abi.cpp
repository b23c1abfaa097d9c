// C ABI of the block-sparse attention library: host-side validation, workspace
// sizing and dispatch to the HIP kernels. No HIP runtime call is made before an
// argument set has been validated, so every error status is returned without
// touching the device (this is also what lets the validation be exercised on a
// machine without a GPU).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/bsa.h"
#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

bsa_status fail(bsa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

bsa_status ok() {
  g_err[0] = '\0';
  return BSA_OK;
}

// Validate a layout and fill the device-side description.
bsa_status make_lay(const bsa_layout* in, bsa::Lay* L) {
  if (!in) return fail(BSA_INVALID_ARG, "layout is NULL");
  for (int a = 0; a < 3; ++a) {
    if (in->grid[a] < 1) return fail(BSA_INVALID_ARG, "grid[%d] = %d must be >= 1", a, in->grid[a]);
    if (in->zone[a] < 1) return fail(BSA_INVALID_ARG, "zone[%d] = %d must be >= 1", a, in->zone[a]);
    if (in->grid[a] > (1 << 20)) return fail(BSA_LAYOUT, "grid[%d] too large", a);
  }
  if (in->mode != BSA_MODE_FIXED && in->mode != BSA_MODE_DYNAMIC)
    return fail(BSA_INVALID_ARG, "mode %d is neither fixed nor dynamic", in->mode);
  if (in->n_shapes < 1 || in->n_shapes > BSA_MAX_SHAPES)
    return fail(BSA_INVALID_ARG, "n_shapes = %d out of [1, %d]", in->n_shapes, BSA_MAX_SHAPES);
  if (in->mode == BSA_MODE_FIXED) {
    if (in->n_shapes != 1) return fail(BSA_LAYOUT, "fixed mode takes exactly one shape");
    for (int a = 0; a < 3; ++a)
      if (in->shapes[0][a] != in->zone[a])
        return fail(BSA_LAYOUT, "fixed mode: zone must equal the block shape");
  }
  const long long ztok = (long long)in->zone[0] * in->zone[1] * in->zone[2];
  long long B = -1;
  for (int s = 0; s < in->n_shapes; ++s) {
    long long b = 1;
    for (int a = 0; a < 3; ++a) {
      const int e = in->shapes[s][a];
      if (e < 1) return fail(BSA_INVALID_ARG, "shape %d axis %d = %d must be >= 1", s, a, e);
      if (in->zone[a] % e)
        return fail(BSA_LAYOUT, "shape %d does not tile the zone on axis %d", s, a);
      b *= e;
    }
    if (B < 0) B = b;
    if (b != B) return fail(BSA_LAYOUT, "candidate shapes must hold the same number of tokens");
  }
  if (B != 64 && B != 128)
    return fail(BSA_UNSUPPORTED, "block of %lld tokens; 64 or 128 supported", B);
  bsa::Lay& o = *L;
  o.T = in->grid[0];
  o.H = in->grid[1];
  o.W = in->grid[2];
  o.zt = in->zone[0];
  o.zh = in->zone[1];
  o.zw = in->zone[2];
  o.gzt = (o.T + o.zt - 1) / o.zt;
  o.gzh = (o.H + o.zh - 1) / o.zh;
  o.gzw = (o.W + o.zw - 1) / o.zw;
  o.n_shapes = in->n_shapes;
  for (int s = 0; s < BSA_MAX_SHAPES; ++s)
    for (int a = 0; a < 3; ++a) o.sh[s][a] = s < in->n_shapes ? in->shapes[s][a] : 1;
  o.B = (int)B;
  o.bpz = (int)(ztok / B);
  const long long nZ = (long long)o.gzt * o.gzh * o.gzw;
  const long long M = nZ * o.bpz;
  if (M > BSA_MAX_BLOCKS)
    return fail(BSA_LAYOUT, "%lld blocks exceed the limit of %d", M, BSA_MAX_BLOCKS);
  o.nZ = (int)nZ;
  o.M = (int)M;
  o.N = (long long)o.T * o.H * o.W;
  o.Np = M * B;
  return ok();
}

bsa_status check_dtype_d(int dtype, int d) {
  if (dtype != BSA_F32 && dtype != BSA_BF16) return fail(BSA_INVALID_ARG, "dtype %d unknown", dtype);
  if (d <= 0) return fail(BSA_INVALID_ARG, "d = %d must be positive", d);
  return ok();
}

bsa_status check_heads(int heads) {
  if (heads < 1 || heads > 65535) return fail(BSA_INVALID_ARG, "heads = %d out of [1, 65535]", heads);
  return ok();
}

size_t esize(int dtype) { return dtype == BSA_BF16 ? 2 : 4; }

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t select_ws(const bsa::Lay& L, int heads) {
  return al256((size_t)heads * L.M * L.M * sizeof(double)) +
         al256((size_t)L.M * sizeof(bsa::BlockMeta));
}

size_t pool_select_ws(const bsa::Lay& L, int heads, int d) {
  return 2 * al256((size_t)heads * L.M * d * sizeof(double)) + select_ws(L, heads);
}

bsa_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(BSA_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

#define BSA_TRY(x)                    \
  do {                                \
    const bsa_status s_ = (x);        \
    if (s_ != BSA_OK) return s_;      \
  } while (0)

}  // namespace

extern "C" {

int bsa_abi_version(void) { return BSA_ABI_VERSION; }

const char* bsa_status_string(bsa_status s) {
  switch (s) {
    case BSA_OK: return "BSA_OK";
    case BSA_INVALID_ARG: return "BSA_INVALID_ARG";
    case BSA_UNSUPPORTED: return "BSA_UNSUPPORTED";
    case BSA_WORKSPACE_TOO_SMALL: return "BSA_WORKSPACE_TOO_SMALL";
    case BSA_LAYOUT: return "BSA_LAYOUT";
    case BSA_HIP_ERROR: return "BSA_HIP_ERROR";
  }
  return "BSA_UNKNOWN_STATUS";
}

const char* bsa_last_error(void) { return g_err; }

bsa_status bsa_layout_sizes(const bsa_layout* in, int64_t* n_tokens, int64_t* n_padded,
                            int32_t* n_blocks, int32_t* n_zones, int32_t* block_tokens) {
  bsa::Lay L;
  BSA_TRY(make_lay(in, &L));
  if (n_tokens) *n_tokens = L.N;
  if (n_padded) *n_padded = L.Np;
  if (n_blocks) *n_blocks = L.M;
  if (n_zones) *n_zones = L.nZ;
  if (block_tokens) *block_tokens = L.B;
  return ok();
}

size_t bsa_workspace_size(bsa_call call, const bsa_layout* in, int heads, int d) {
  bsa::Lay L;
  if (make_lay(in, &L) != BSA_OK) return 0;
  if (heads < 1) heads = 1;
  if (d < 1) d = 1;
  switch (call) {
    case BSA_CALL_ZONE_SCORE: return bsa::zone_score_workspace(L, d, 256);
    case BSA_CALL_POOL_SELECT: return pool_select_ws(L, heads, d);
    case BSA_CALL_ATTN_FWD: return bsa::attn_fwd_workspace(L, d, true);
    case BSA_CALL_ATTN_BWD: return bsa::attn_bwd_workspace(L, heads, d);
    case BSA_CALL_SELECT: return select_ws(L, heads);
  }
  fail(BSA_INVALID_ARG, "unknown call %d", (int)call);
  return 0;
}

bsa_status bsa_zone_score(const bsa_layout* in, const void* video, int C, const void* audio,
                          int n_audio, int32_t* zone_shape, double* zone_stats, void* ws,
                          size_t ws_bytes, void* stream) {
  bsa::Lay L;
  BSA_TRY(make_lay(in, &L));
  if (!zone_shape) return fail(BSA_INVALID_ARG, "zone_shape is NULL");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (in->mode == BSA_MODE_FIXED)
    return hip_status(bsa::launch_zone_score(L, nullptr, 0, nullptr, 0, zone_shape, nullptr,
                                             nullptr, st),
                      "zone_score");
  if (!video) return fail(BSA_INVALID_ARG, "video is NULL in dynamic mode");
  if (C < 64 || C > 8192 || C % 64) return fail(BSA_INVALID_ARG, "C = %d must be a multiple of 64 in [64, 8192]", C);
  if ((audio == nullptr) != (n_audio == 0))
    return fail(BSA_INVALID_ARG, "audio and n_audio must both be given or both absent");
  if (n_audio < 0 || n_audio > 256) return fail(BSA_INVALID_ARG, "n_audio = %d out of [0, 256]", n_audio);
  if (L.zt > 4 || L.zh > 16 || L.zw > 16)
    return fail(BSA_UNSUPPORTED, "zone scoring supports zones up to 4x16x16");
  if ((long long)L.zt * L.H * L.W * C * 2 >= (1LL << 31))
    return fail(BSA_UNSUPPORTED, "zone scoring needs zt*H*W*C*2 < 2^31 (one zone's offsets in 32 bits)");
  const size_t need = bsa::zone_score_workspace(L, C, n_audio);
  if (!ws || ws_bytes < need)
    return fail(BSA_WORKSPACE_TOO_SMALL, "zone_score needs %zu workspace bytes, got %zu", need, ws_bytes);
  return hip_status(bsa::launch_zone_score(L, video, C, audio, n_audio, zone_shape, zone_stats,
                                           ws, st),
                    "zone_score");
}

static bsa_status permute_common(const bsa_layout* in, const int32_t* zone_shape, int ntensors,
                                 const void* const* src, void* const* dst, int heads, int d,
                                 int dtype, void* stream, bool inverse, int npool = 0,
                                 double* const* means = nullptr, int nrope = 0,
                                 const float* const* gamma = nullptr, float eps = 0.f,
                                 float rope_base = 0.f) {
  bsa::Lay L;
  BSA_TRY(make_lay(in, &L));
  BSA_TRY(check_heads(heads));
  BSA_TRY(check_dtype_d(dtype, d));
  if (ntensors < 1 || ntensors > 4) return fail(BSA_INVALID_ARG, "ntensors = %d out of [1, 4]", ntensors);
  if (!src || !dst) return fail(BSA_INVALID_ARG, "src/dst pointer arrays are NULL");
  // a pooled tensor may have no dst (bsa_permute_pool only): it is read and
  // pooled, and its gathered copy is not stored
  for (int i = 0; i < ntensors; ++i)
    if (!src[i] || (!dst[i] && (inverse || nrope > 0 || i >= npool)))
      return fail(BSA_INVALID_ARG, "tensor %d pointer is NULL", i);
  for (int i = 0; i < ntensors; ++i)
    if (reinterpret_cast<uintptr_t>(src[i]) % 16 || reinterpret_cast<uintptr_t>(dst[i]) % 16)
      return fail(BSA_INVALID_ARG, "tensor %d: src and dst must be 16-byte aligned", i);
  const size_t row = (size_t)d * esize(dtype);
  if (row % 16 || d > 256) return fail(BSA_UNSUPPORTED, "row of %zu bytes (d = %d); need a multiple of 16 bytes and d <= 256", row, d);
  if (in->mode == BSA_MODE_DYNAMIC && !zone_shape)
    return fail(BSA_INVALID_ARG, "zone_shape is NULL in dynamic mode");
  if (npool < 0 || npool > ntensors) return fail(BSA_INVALID_ARG, "npool = %d out of [0, %d]", npool, ntensors);
  if (nrope < 0 || nrope > ntensors) return fail(BSA_INVALID_ARG, "nrope = %d out of [0, %d]", nrope, ntensors);
  if (nrope > 0) {
    if (d != 64 && d != 128) return fail(BSA_UNSUPPORTED, "norm + RoPE needs d in {64, 128}, got %d", d);
    if (!(eps > 0.f) || isinf(eps)) return fail(BSA_INVALID_ARG, "eps = %g must be finite and > 0", (double)eps);
    if (!(rope_base > 1.f) || isinf(rope_base))
      return fail(BSA_INVALID_ARG, "rope_base = %g must be finite and > 1", (double)rope_base);
  }
  if (npool > 0) {
    if (d != 64 && d != 128) return fail(BSA_UNSUPPORTED, "pooling needs d in {64, 128}, got %d", d);
    if (!means) return fail(BSA_INVALID_ARG, "means pointer array is NULL");
    for (int i = 0; i < npool; ++i)
      if (!means[i]) return fail(BSA_INVALID_ARG, "means %d pointer is NULL", i);
  }
  return hip_status(bsa::launch_permute(L, zone_shape, ntensors, src, dst, heads, (int)row,
                                        inverse, static_cast<hipStream_t>(stream), npool, means,
                                        dtype == BSA_BF16 ? 8 : 4, nrope, gamma, eps, rope_base),
                    inverse ? "unpermute" : "permute");
}

bsa_status bsa_permute_norm_rope(const bsa_layout* in, const int32_t* zone_shape, int ntensors,
                                 const void* const* src, void* const* dst, int heads, int d,
                                 int dtype, int nrope, const float* const* gamma, float eps,
                                 float rope_base, int npool, double* const* means, void* stream) {
  return permute_common(in, zone_shape, ntensors, src, dst, heads, d, dtype, stream, false,
                        npool, means, nrope, gamma, eps, rope_base);
}

bsa_status bsa_permute_pool(const bsa_layout* in, const int32_t* zone_shape, int ntensors,
                            const void* const* src, void* const* dst, int heads, int d,
                            int dtype, int npool, double* const* means, void* stream) {
  return permute_common(in, zone_shape, ntensors, src, dst, heads, d, dtype, stream, false,
                        npool, means);
}

bsa_status bsa_permute(const bsa_layout* in, const int32_t* zone_shape, int ntensors,
                       const void* const* src, void* const* dst, int heads, int d, int dtype,
                       void* stream) {
  return permute_common(in, zone_shape, ntensors, src, dst, heads, d, dtype, stream, false);
}

bsa_status bsa_unpermute(const bsa_layout* in, const int32_t* zone_shape, int ntensors,
                         const void* const* src, void* const* dst, int heads, int d, int dtype,
                         void* stream) {
  return permute_common(in, zone_shape, ntensors, src, dst, heads, d, dtype, stream, true);
}

static bsa_status check_select_args(const bsa_layout* in, const bsa::Lay& L,
                                    const int32_t* zone_shape, int heads, int d,
                                    int32_t sparsity_1e4, double tau, const void* counts,
                                    const void* idx) {
  (void)L;
  BSA_TRY(check_heads(heads));
  if (d != 64 && d != 128) return fail(BSA_UNSUPPORTED, "d = %d; 64 or 128 supported", d);
  if (!counts || !idx) return fail(BSA_INVALID_ARG, "counts/idx is NULL");
  if (in->mode == BSA_MODE_DYNAMIC && !zone_shape)
    return fail(BSA_INVALID_ARG, "zone_shape is NULL in dynamic mode");
  if (sparsity_1e4 < 0 || sparsity_1e4 > 9999)
    return fail(BSA_INVALID_ARG, "sparsity_1e4 = %d out of [0, 9999]", sparsity_1e4);
  if (!(tau > 0.0 && tau <= 1.0)) return fail(BSA_INVALID_ARG, "tau = %g out of (0, 1]", tau);
  return ok();
}

// block facts, pooled logits and selection from block means (p: select_ws bytes)
static hipError_t select_tail(const bsa::Lay& L, const int32_t* zone_shape, const double* qbar,
                              const double* kbar, int heads, int d, int32_t sparsity_1e4,
                              double tau, int32_t* counts, int32_t* idx, double* pooled_logits,
                              char* p, hipStream_t st, bool meta_ready,
                              int frames_per_chunk = 0) {
  double* logits = pooled_logits ? pooled_logits : reinterpret_cast<double*>(p);
  p += al256((size_t)heads * L.M * L.M * sizeof(double));
  bsa::BlockMeta* meta = reinterpret_cast<bsa::BlockMeta*>(p);
  hipError_t e = meta_ready ? hipSuccess : bsa::launch_block_meta(L, zone_shape, meta, st);
  if (e == hipSuccess)
    e = bsa::launch_pooled_logits(L, meta, qbar, kbar, heads, d, 1.0 / sqrt((double)d), logits,
                                  st);
  if (e == hipSuccess)
    e = bsa::launch_select(L, meta, logits, heads, sparsity_1e4, tau, counts, idx, st,
                           frames_per_chunk);
  return e;
}

bsa_status bsa_pool_select(const bsa_layout* in, const int32_t* zone_shape, const void* qp,
                           const void* kp, int heads, int d, int dtype, int32_t sparsity_1e4,
                           double tau, int32_t* counts, int32_t* idx, double* pooled_logits,
                           void* ws, size_t ws_bytes, void* stream) {
  bsa::Lay L;
  BSA_TRY(make_lay(in, &L));
  BSA_TRY(check_dtype_d(dtype, d));
  BSA_TRY(check_select_args(in, L, zone_shape, heads, d, sparsity_1e4, tau, counts, idx));
  if (!qp || !kp) return fail(BSA_INVALID_ARG, "qp/kp is NULL");
  const size_t need = pool_select_ws(L, heads, d);
  if (!ws || ws_bytes < need)
    return fail(BSA_WORKSPACE_TOO_SMALL, "pool_select needs %zu workspace bytes, got %zu", need, ws_bytes);
  char* p = static_cast<char*>(ws);
  double* qbar = reinterpret_cast<double*>(p);
  p += al256((size_t)heads * L.M * d * sizeof(double));
  double* kbar = reinterpret_cast<double*>(p);
  p += al256((size_t)heads * L.M * d * sizeof(double));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  bsa::BlockMeta* meta = reinterpret_cast<bsa::BlockMeta*>(
      p + al256((size_t)heads * L.M * L.M * sizeof(double)));
  hipError_t e = bsa::launch_block_meta(L, zone_shape, meta, st);
  if (e == hipSuccess)
    e = bsa::launch_pool(L, meta, qp, kp, heads, d, dtype == BSA_BF16, qbar, kbar, st);
  if (e == hipSuccess)
    e = select_tail(L, zone_shape, qbar, kbar, heads, d, sparsity_1e4, tau, counts, idx,
                    pooled_logits, p, st, true);
  return hip_status(e, "pool_select");
}

static bsa_status select_common(const bsa_layout* in, const int32_t* zone_shape,
                                const double* qbar, const double* kbar, int heads, int d,
                                int32_t sparsity_1e4, double tau, int frames_per_chunk,
                                int32_t* counts, int32_t* idx, double* pooled_logits, void* ws,
                                size_t ws_bytes, void* stream) {
  bsa::Lay L;
  BSA_TRY(make_lay(in, &L));
  BSA_TRY(check_select_args(in, L, zone_shape, heads, d, sparsity_1e4, tau, counts, idx));
  if (!qbar || !kbar) return fail(BSA_INVALID_ARG, "qbar/kbar is NULL");
  if (frames_per_chunk < 0 || (frames_per_chunk > 0 && frames_per_chunk % L.zt))
    return fail(BSA_INVALID_ARG, "frames_per_chunk = %d must be a positive multiple of the zone's time extent %d",
                frames_per_chunk, L.zt);
  const size_t need = select_ws(L, heads);
  if (!ws || ws_bytes < need)
    return fail(BSA_WORKSPACE_TOO_SMALL, "select needs %zu workspace bytes, got %zu", need, ws_bytes);
  return hip_status(select_tail(L, zone_shape, qbar, kbar, heads, d, sparsity_1e4, tau, counts,
                                idx, pooled_logits, static_cast<char*>(ws),
                                static_cast<hipStream_t>(stream), false, frames_per_chunk),
                    "select");
}

bsa_status bsa_select(const bsa_layout* in, const int32_t* zone_shape, const double* qbar,
                      const double* kbar, int heads, int d, int32_t sparsity_1e4, double tau,
                      int32_t* counts, int32_t* idx, double* pooled_logits, void* ws,
                      size_t ws_bytes, void* stream) {
  return select_common(in, zone_shape, qbar, kbar, heads, d, sparsity_1e4, tau, 0, counts, idx,
                       pooled_logits, ws, ws_bytes, stream);
}

bsa_status bsa_select_causal(const bsa_layout* in, const int32_t* zone_shape, const double* qbar,
                             const double* kbar, int heads, int d, int32_t sparsity_1e4,
                             double tau, int frames_per_chunk, int32_t* counts, int32_t* idx,
                             double* pooled_logits, void* ws, size_t ws_bytes, void* stream) {
  if (frames_per_chunk < 1)
    return fail(BSA_INVALID_ARG, "frames_per_chunk = %d must be >= 1", frames_per_chunk);
  return select_common(in, zone_shape, qbar, kbar, heads, d, sparsity_1e4, tau,
                       frames_per_chunk, counts, idx, pooled_logits, ws, ws_bytes, stream);
}

static bsa_status attn_fwd_common(const bsa_layout* in, const int32_t* zone_shape,
                                  const void* qp, const void* kp, const void* vp,
                                  const int32_t* counts, const int32_t* idx, int heads, int d,
                                  int dtype, float scale, void* op, float* lse, void* ws,
                                  size_t ws_bytes, void* stream, bool raster,
                                  bool static_scratch = false, bool gather = false) {
  bsa::Lay L;
  BSA_TRY(make_lay(in, &L));
  BSA_TRY(check_heads(heads));
  BSA_TRY(check_dtype_d(dtype, d));
  if (d != 64 && d != 128) return fail(BSA_UNSUPPORTED, "d = %d; 64 or 128 supported", d);
  if (raster && !bsa::attn_fwd_uses_mfma(L, d, dtype == BSA_BF16))
    return fail(BSA_UNSUPPORTED, "raster output needs bf16, d = 128 and 128-token blocks");
  if (gather && !bsa::attn_fwd_gather_ok(L, d, dtype == BSA_BF16))
    return fail(BSA_UNSUPPORTED, "the gathered forward needs bf16, d = 128, 128-token blocks, "
                "block widths that are multiples of 4 and Np * 256 < 2^31");
  if (!qp || !kp || !vp || !counts || !idx || !op || !lse)
    return fail(BSA_INVALID_ARG, "a tensor pointer is NULL");
  for (const void* p : {qp, kp, vp, static_cast<const void*>(op)})
    if (reinterpret_cast<uintptr_t>(p) % 16)
      return fail(BSA_INVALID_ARG, "qp, kp, vp and the output must be 16-byte aligned");
  if (in->mode == BSA_MODE_DYNAMIC && !zone_shape)
    return fail(BSA_INVALID_ARG, "zone_shape is NULL in dynamic mode");
  if (!(scale >= 0.f) || isinf(scale)) return fail(BSA_INVALID_ARG, "scale must be finite and >= 0");
  const size_t need = bsa::attn_fwd_workspace(L, d, dtype == BSA_BF16);
  if (static_scratch) {
    // the library's own scratch array replaces the caller's workspace
    size_t have = 0;
    const hipError_t e = bsa::attn_fwd_static_scratch(&ws, &have);
    if (e != hipSuccess) return hip_status(e, "attn_fwd_noalloc scratch lookup");
    if (need > have)
      return fail(BSA_LAYOUT, "attn_fwd_noalloc: the block table needs %zu bytes, its static "
                  "scratch holds %zu", need, have);
    ws_bytes = have;
  }
  if (need && (!ws || ws_bytes < need))
    return fail(BSA_WORKSPACE_TOO_SMALL, "attn_fwd needs %zu workspace bytes, got %zu", need, ws_bytes);
  const float sc = scale == 0.f ? 1.0f / sqrtf((float)d) : scale;
  return hip_status(bsa::launch_attn_fwd(L, zone_shape, qp, kp, vp, counts, idx, heads, d,
                                         dtype == BSA_BF16, sc, op, lse, ws,
                                         static_cast<hipStream_t>(stream), raster, gather),
                    "attn_fwd");
}

bsa_status bsa_attn_fwd(const bsa_layout* in, const int32_t* zone_shape, const void* qp,
                        const void* kp, const void* vp, const int32_t* counts,
                        const int32_t* idx, int heads, int d, int dtype, float scale, void* op,
                        float* lse, void* ws, size_t ws_bytes, void* stream) {
  return attn_fwd_common(in, zone_shape, qp, kp, vp, counts, idx, heads, d, dtype, scale, op,
                         lse, ws, ws_bytes, stream, false);
}

bsa_status bsa_attn_fwd_noalloc(const bsa_layout* in, const int32_t* zone_shape, const void* qp,
                                const void* kp, const void* vp, const int32_t* counts,
                                const int32_t* idx, int heads, int d, int dtype, float scale,
                                void* op, float* lse, void* stream) {
  return attn_fwd_common(in, zone_shape, qp, kp, vp, counts, idx, heads, d, dtype, scale, op,
                         lse, nullptr, 0, stream, false, true);
}

bsa_status bsa_attn_fwd_raster(const bsa_layout* in, const int32_t* zone_shape, const void* qp,
                               const void* kp, const void* vp, const int32_t* counts,
                               const int32_t* idx, int heads, int d, int dtype, float scale,
                               void* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return attn_fwd_common(in, zone_shape, qp, kp, vp, counts, idx, heads, d, dtype, scale, o,
                         lse, ws, ws_bytes, stream, true);
}

bsa_status bsa_attn_fwd_gather(const bsa_layout* in, const int32_t* zone_shape, const void* q,
                               const void* k, const void* v, const int32_t* counts,
                               const int32_t* idx, int heads, int d, int dtype, float scale,
                               void* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return attn_fwd_common(in, zone_shape, q, k, v, counts, idx, heads, d, dtype, scale, o, lse, ws,
                         ws_bytes, stream, true, false, true);
}

static bsa_status attn_bwd_common(const bsa_layout* in, const int32_t* zone_shape,
                                  const void* qp, const void* kp, const void* vp, const void* op,
                                  const void* dop, const float* lse, const int32_t* counts,
                                  const int32_t* idx, int heads, int d, int dtype, float scale,
                                  void* dqp, void* dkp, void* dvp, void* ws, size_t ws_bytes,
                                  void* stream, bool raster) {
  bsa::Lay L;
  BSA_TRY(make_lay(in, &L));
  BSA_TRY(check_heads(heads));
  BSA_TRY(check_dtype_d(dtype, d));
  if (d != 64 && d != 128) return fail(BSA_UNSUPPORTED, "d = %d; 64 or 128 supported", d);
  if (raster && !bsa::attn_fwd_uses_mfma(L, d, dtype == BSA_BF16))
    return fail(BSA_UNSUPPORTED, "raster gradients need bf16, d = 128 and 128-token blocks");
  if (!qp || !kp || !vp || !op || !dop || !lse || !counts || !idx || !dqp || !dkp || !dvp)
    return fail(BSA_INVALID_ARG, "a tensor pointer is NULL");
  for (const void* p : {qp, kp, vp, op, dop})
    if (reinterpret_cast<uintptr_t>(p) % 16)
      return fail(BSA_INVALID_ARG, "qp, kp, vp, op, dop must be 16-byte aligned");
  if (in->mode == BSA_MODE_DYNAMIC && !zone_shape)
    return fail(BSA_INVALID_ARG, "zone_shape is NULL in dynamic mode");
  if (!(scale >= 0.f) || isinf(scale)) return fail(BSA_INVALID_ARG, "scale must be finite and >= 0");
  const size_t need = bsa::attn_bwd_workspace(L, heads, d);
  if (!ws || ws_bytes < need)
    return fail(BSA_WORKSPACE_TOO_SMALL, "attn_bwd needs %zu workspace bytes, got %zu", need, ws_bytes);
  const float sc = scale == 0.f ? 1.0f / sqrtf((float)d) : scale;
  return hip_status(bsa::launch_attn_bwd(L, zone_shape, qp, kp, vp, op, dop, lse, counts, idx,
                                         heads, d, dtype == BSA_BF16, sc, dqp, dkp, dvp, ws,
                                         static_cast<hipStream_t>(stream), raster),
                    "attn_bwd");
}

bsa_status bsa_attn_bwd(const bsa_layout* in, const int32_t* zone_shape, const void* qp,
                        const void* kp, const void* vp, const void* op, const void* dop,
                        const float* lse, const int32_t* counts, const int32_t* idx, int heads,
                        int d, int dtype, float scale, void* dqp, void* dkp, void* dvp,
                        void* ws, size_t ws_bytes, void* stream) {
  return attn_bwd_common(in, zone_shape, qp, kp, vp, op, dop, lse, counts, idx, heads, d, dtype,
                         scale, dqp, dkp, dvp, ws, ws_bytes, stream, false);
}

bsa_status bsa_attn_bwd_raster(const bsa_layout* in, const int32_t* zone_shape, const void* qp,
                               const void* kp, const void* vp, const void* op, const void* dop,
                               const float* lse, const int32_t* counts, const int32_t* idx,
                               int heads, int d, int dtype, float scale, void* dq, void* dk,
                               void* dv, void* ws, size_t ws_bytes, void* stream) {
  return attn_bwd_common(in, zone_shape, qp, kp, vp, op, dop, lse, counts, idx, heads, d, dtype,
                         scale, dq, dk, dv, ws, ws_bytes, stream, true);
}

}  // extern "C"

static bsa_status check_xattn(int n_video, int n_audio, int C, int heads, int d) {
  if (n_video < 1) return fail(BSA_INVALID_ARG, "n_video = %d must be >= 1", n_video);
  if (n_audio < 1 || n_audio > 256) return fail(BSA_INVALID_ARG, "n_audio = %d out of [1, 256]", n_audio);
  if (C < 64 || C > 8192 || C % 64) return fail(BSA_INVALID_ARG, "C = %d must be a multiple of 64 in [64, 8192]", C);
  if (heads < 1 || heads > 64) return fail(BSA_INVALID_ARG, "heads = %d out of [1, 64]", heads);
  if (d != 128) return fail(BSA_UNSUPPORTED, "d = %d; the cross-attention supports d = 128", d);
  return ok();
}

bsa_status bsa_xattn_fwd(int n_video, int n_audio, int C, int heads, int d, const void* x,
                         const void* a, const void* wq, const void* wk, const void* wv,
                         const void* wo, void* q, void* k, void* v, void* o, float* lse, void* y,
                         void* stream) {
  BSA_TRY(check_xattn(n_video, n_audio, C, heads, d));
  const void* in[] = {x, a, wq, wk, wv, wo, q, k, v, o, lse, y};
  for (const void* p : in)
    if (!p) return fail(BSA_INVALID_ARG, "a tensor pointer is NULL");
  for (const void* p : in)
    if (reinterpret_cast<uintptr_t>(p) % 16) return fail(BSA_INVALID_ARG, "tensors must be 16-byte aligned");
  typedef const __bf16* cb;
  return hip_status(bsa::launch_xattn_fwd(n_video, n_audio, heads, (cb)x, (cb)a, C, (cb)wq, (cb)wk,
                                          (cb)wv, (cb)wo, (__bf16*)q, (__bf16*)k, (__bf16*)v,
                                          (__bf16*)o, lse, (__bf16*)y,
                                          static_cast<hipStream_t>(stream)),
                    "xattn_fwd");
}

size_t bsa_xattn_bwd_workspace_size(int n_video, int n_audio, int C, int heads) {
  if (check_xattn(n_video, n_audio, C, heads, 128) != BSA_OK) return 0;
  return bsa::xattn_bwd_workspace(n_video, n_audio, C, heads);
}

bsa_status bsa_xattn_bwd(int n_video, int n_audio, int C, int heads, int d, const void* x,
                         const void* a, const void* wq, const void* wk, const void* wv,
                         const void* wo, const void* q, const void* k, const void* v,
                         const void* o, const float* lse, const void* dy, float* dx, float* da,
                         float* dwq, float* dwk, float* dwv, float* dwo, void* ws,
                         size_t ws_bytes, void* stream) {
  BSA_TRY(check_xattn(n_video, n_audio, C, heads, d));
  const void* in[] = {x, a, wq, wk, wv, wo, q, k, v, o, lse, dy, dx, da, dwq, dwk, dwv, dwo};
  for (const void* p : in)
    if (!p) return fail(BSA_INVALID_ARG, "a tensor pointer is NULL");
  for (const void* p : in)
    if (reinterpret_cast<uintptr_t>(p) % 16) return fail(BSA_INVALID_ARG, "tensors must be 16-byte aligned");
  const size_t need = bsa::xattn_bwd_workspace(n_video, n_audio, C, heads);
  if (!ws || ws_bytes < need)
    return fail(BSA_WORKSPACE_TOO_SMALL, "xattn_bwd needs %zu workspace bytes, got %zu", need, ws_bytes);
  if (reinterpret_cast<uintptr_t>(ws) % 16)
    return fail(BSA_INVALID_ARG, "the workspace must be 16-byte aligned");
  typedef const __bf16* cb;
  return hip_status(bsa::launch_xattn_bwd(n_video, n_audio, heads, (cb)x, (cb)a, C, (cb)wq,
                                          (cb)wk, (cb)wv, (cb)wo, (cb)q, (cb)k, (cb)v, (cb)o, lse,
                                          (cb)dy, dx, da, dwq, dwk, dwv, dwo, ws,
                                          static_cast<hipStream_t>(stream)),
                    "xattn_bwd");
}

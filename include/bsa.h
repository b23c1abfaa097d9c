/*
 * bsa.h -- C ABI of the MI355X (gfx950) block-sparse attention library.
 *
 * The method: Prism block sparse attention (BSA), described on the page
 * "Prism: 2K 공동 영상·오디오 생성 학습을 위한 동적 희소 어텐션" (Prism: dynamic
 * sparse attention for training 2K joint video-audio generation;
 * trawling.dev/post/2299), section "지역별 정보에 맞춘 블록 구성" (block
 * composition matched to regional information), cited below as [Prism §Blocks].
 * Latent tokens are split into spatio-temporal macro-zones; each zone picks a
 * block shape from the channel-wise variance of the video features and the
 * audio-to-video cross-attention feature norm; tokens are regrouped into those
 * blocks; key blocks are selected per query block by a hybrid rule (a top-k
 * set from a sparsity value, united with the smallest CDF prefix reaching a
 * threshold tau, 0.20 in the page's configuration); attention then runs over
 * the selected blocks only. The page gives no formulas; the exact reading
 * implemented here is stated at each call.
 *
 * Conventions shared by every call
 * --------------------------------
 * Memory.   Pointers are device pointers unless marked [host]. The caller
 *           allocates every device buffer, including the workspace; the
 *           library never allocates or frees memory, keeps no pointer after a
 *           call returns, and has no global mutable state (thread-safe).
 * Streams.  `stream` is a hipStream_t (NULL = the default stream). A call only
 *           enqueues kernels on it: it never synchronizes and never copies
 *           between host and device.
 * Errors.   Every call returns a bsa_status. All arguments are validated on
 *           the host before the first launch, so a call that returns an error
 *           status has launched nothing and written nothing. bsa_last_error()
 *           gives a thread-local message for the last failure. Faults inside a
 *           kernel surface at the caller's next synchronization (HIP semantics).
 * Tokens.   Q/K/V are [heads, tokens, d], row-major, token id raster over the
 *           latent grid with t slowest: n = (t*H + h)*W + w.
 * Layout.   Each grid axis is padded up to a multiple of the zone extent.
 *           Zones are ordered raster over the zone grid; inside a zone, blocks
 *           are raster over its (zt/bt, zh/bh, zw/bw) sub-grid; inside a block,
 *           tokens are raster. Block b covers slots [b*B, (b+1)*B) of the
 *           permuted ("padded") token axis, B = bt*bh*bw. A slot is real iff
 *           its (t,h,w) lies inside the grid; pad slots hold zeros.
 * Dtypes.   BSA_BF16 is the performance path; BSA_F32 is the exact-parity path.
 */
#ifndef BSA_H_
#define BSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSA_ABI_VERSION 1
#define BSA_MAX_SHAPES 4
#define BSA_MAX_BLOCKS 4096   /* per layout: one selection row lives in one wavefront's registers, and the attention block lists are staged in LDS */

typedef enum {
  BSA_OK = 0,
  BSA_INVALID_ARG = 1,         /* null pointer, non-positive size, value out of range */
  BSA_UNSUPPORTED = 2,         /* dtype / head dim / block size the library has no kernel for */
  BSA_WORKSPACE_TOO_SMALL = 3, /* ws_bytes < bsa_workspace_size(...) */
  BSA_LAYOUT = 4,              /* a shape does not tile the zone, too many blocks, ... */
  BSA_HIP_ERROR = 5            /* a kernel launch failed */
} bsa_status;

typedef enum { BSA_F32 = 0, BSA_BF16 = 1 } bsa_dtype;
typedef enum { BSA_MODE_FIXED = 0, BSA_MODE_DYNAMIC = 1 } bsa_mode;

/* Which call a workspace is sized for. */
typedef enum {
  BSA_CALL_ZONE_SCORE = 0,
  BSA_CALL_POOL_SELECT = 1,
  BSA_CALL_ATTN_FWD = 2,
  BSA_CALL_ATTN_BWD = 3,
  BSA_CALL_SELECT = 4
} bsa_call;

/* [host] Description of the token layout (plain data, read during a call only).
 *  grid    latent grid (T, H, W), each >= 1
 *  mode    BSA_MODE_FIXED: one block shape everywhere; `zone` must equal
 *          shapes[0] and n_shapes must be 1 (each zone is one block).
 *          BSA_MODE_DYNAMIC: `zone` is the macro-zone extent (4,16,16 on the
 *          measured workloads) and shapes[0..n_shapes) are the candidate block
 *          shapes in canonical order (shape id = index; the measured workloads
 *          use 0 = 2x8x8, 1 = 4x4x8, 2 = 1x8x16).
 *  Every shape must divide the zone on each axis and hold B tokens, the same
 *  B for all shapes; B must be 64 or 128. */
typedef struct bsa_layout {
  int32_t grid[3];
  int32_t mode;
  int32_t zone[3];
  int32_t n_shapes;
  int32_t shapes[BSA_MAX_SHAPES][3];
} bsa_layout;

/* Library version; equals BSA_ABI_VERSION of the header it was built from. */
int bsa_abi_version(void);

/* Human-readable name of a status code (static storage). */
const char* bsa_status_string(bsa_status s);

/* Thread-local message describing the last non-OK status of this thread. */
const char* bsa_last_error(void);

/* [host only, no device access] Sizes implied by a layout. Any output pointer
 * may be NULL.  n_tokens = T*H*W; n_padded = n_blocks * B; n_blocks = zones *
 * blocks per zone; n_zones = number of macro-zones; block_tokens = B.
 * Returns BSA_LAYOUT / BSA_INVALID_ARG for an invalid layout. */
bsa_status bsa_layout_sizes(const bsa_layout* L, int64_t* n_tokens, int64_t* n_padded,
                            int32_t* n_blocks, int32_t* n_zones, int32_t* block_tokens);

/* [host only] Bytes of device workspace a call needs (0 if none). `heads` and
 * `d` are those the call will receive (ignored by BSA_CALL_ZONE_SCORE, which
 * needs `d` = the video channel count C instead). Returns 0 and sets the last
 * error for an invalid layout; check bsa_last_error() when 0 is unexpected. */
size_t bsa_workspace_size(bsa_call call, const bsa_layout* L, int heads, int d);

/* Zone scoring and block-shape choice [Prism §Blocks: per macro-zone, the
 * channel-wise variance of the video features and the A2V cross-attention
 * feature norm set the zone's block shape; axes with fast change or strong
 * audio-video coupling are split more finely].
 * Reading implemented (the page gives no formula):
 *   g_n  = || sum_j softmax_j(X_n . A_j / sqrt(C)) A_j ||   (one head, identity
 *          projections);
 *   V_a(z) = sum over lines along axis a of sum ||X_n - line mean||^2 / (C n_z),
 *   G_a(z) = the same for the scalar g, divided by n_z (lines = the zone's real
 *          tokens sharing the other two coordinates; n_z = real tokens of z);
 *   r_a(z) = V_a(z)/mean(V) + G_a(z)/mean(G), means over non-empty (zone, axis);
 *   shape(z) = argmin_s sum_a r_a(z) (b_{s,a}^2 - 1)/(Z_a^2 - 1); costs within a
 *          relative 1e-6 of the minimum tie and the lowest shape id wins.
 *  video       [N, C] bf16, raster token order, N = T*H*W
 *  C           channels (64..8192, multiple of 64); zones up to 4x16x16 and
 *              zt*H*W*C*2 < 2^31 (BSA_UNSUPPORTED otherwise)
 *  audio       [n_audio, C] bf16, or NULL (then the A2V term is dropped)
 *  n_audio     0..256 (0 iff audio == NULL)
 *  zone_shape  [n_zones] int32 out: shape id per zone
 *  zone_stats  [n_zones, 3, 2] double out (V_t, G_t, V_h, G_h, V_w, G_w per zone), or NULL
 *  In fixed mode the call writes 0 to every zone_shape entry and ignores the
 *  features (video/audio may be NULL). */
bsa_status bsa_zone_score(const bsa_layout* L, const void* video, int C, const void* audio,
                          int n_audio, int32_t* zone_shape, double* zone_stats, void* ws,
                          size_t ws_bytes, void* stream);

/* Gather tokens into block order [Prism §Blocks: tokens are regrouped into the
 * zone's blocks so that a block holds semantically close tokens].
 *  zone_shape  [n_zones] int32 shape ids (device data, so not validated on the
 *              host; an id outside [0, n_shapes) is clamped into it), or NULL
 *              for all zeros (fixed mode)
 *  ntensors    1..4 tensors handled by one launch
 *  src         [host] array of ntensors device pointers, each [heads, N, d]
 *  dst         [host] array of ntensors device pointers, each [heads, Np, d];
 *              pad slots are written with zeros
 *  d           head dim (multiple of 8, <= 256); dtype BSA_F32 or BSA_BF16
 *  Every src and dst pointer must be 16-byte aligned (BSA_INVALID_ARG otherwise). */
bsa_status bsa_permute(const bsa_layout* L, const int32_t* zone_shape, int ntensors,
                       const void* const* src, void* const* dst, int heads, int d, int dtype,
                       void* stream);

/* bsa_permute that also pools [Prism §Blocks: block-level features]: while
 * gathering, it sums the real rows of every block of the first npool tensors
 * in fp64 and writes their means, the q̄ / k̄ that block selection scores
 * (so that selection need not read Qp and Kp again).
 *  npool   0..ntensors tensors to pool (0 = plain bsa_permute)
 *  means   [host] array of npool device pointers, each [heads, n_blocks, d]
 *          double out: mean of the block's real slots (0 for an empty block)
 *  dst     as bsa_permute, except that dst[i] may be NULL for a pooled tensor
 *          (i < npool): it is read and pooled, and no gathered copy is stored
 *          (the path of bsa_attn_fwd_gather, which gathers Q, K, V itself)
 *  Other arguments as bsa_permute; pooling needs d in {64, 128}. */
bsa_status bsa_permute_pool(const bsa_layout* L, const int32_t* zone_shape, int ntensors,
                            const void* const* src, void* const* dst, int heads, int d,
                            int dtype, int npool, double* const* means, void* stream);

/* bsa_permute_pool with the pre-attention transform of Q and K fused into the
 * gather [Helios page (suanlab.com, Helios review), core contributions: fused
 * normalization and RoPE kernels; Kaleido page (gist.science, paper
 * 2607.13770), methodology: the rotary embedding splits a head's channels into
 * a time group and two spatial groups, each at its own frequencies].
 * Reading implemented (the pages give no formula), on each token's head
 * vector of the first nrope tensors, in fp32, rounded once to the dtype:
 *   y = x / sqrt(mean_c x_c^2 + eps) * gamma   (RMSNorm over the d channels);
 *   channel groups t, h, w of d - 4 floor(d/6), 2 floor(d/6), 2 floor(d/6)
 *   channels; the pair (2i, 2i+1) of a group of g channels turns by
 *   pos * rope_base^(-2i/g), pos = the token's t, h or w:
 *   (y0, y1) -> (y0 cos a - y1 sin a, y0 sin a + y1 cos a).
 *  nrope      0..ntensors tensors to transform (Q and K: 2)
 *  gamma      [host] array of nrope device pointers to [d] float weights, or
 *             NULL (all weights 1); a NULL entry means weights 1 for that tensor
 *  eps        > 0;  rope_base > 1 (10000 is usual)
 *  npool/means as in bsa_permute_pool; the means are those of the stored
 *             (transformed, rounded) rows.
 *  Other arguments as bsa_permute; the transform needs d in {64, 128}. */
bsa_status bsa_permute_norm_rope(const bsa_layout* L, const int32_t* zone_shape, int ntensors,
                                 const void* const* src, void* const* dst, int heads, int d,
                                 int dtype, int nrope, const float* const* gamma, float eps,
                                 float rope_base, int npool, double* const* means, void* stream);

/* Inverse of bsa_permute [Prism §Blocks: attention runs on the tokens
 * regrouped into the zones' blocks, so its outputs (and, in training, its
 * gradients) are in block order and go back to the latent token order the rest
 * of the model uses]: src [heads, Np, d] -> dst [heads, N, d], reading real
 * slots only (pad slots are dropped). Same arguments as bsa_permute; src and
 * dst 16-byte aligned. */
bsa_status bsa_unpermute(const bsa_layout* L, const int32_t* zone_shape, int ntensors,
                         const void* const* src, void* const* dst, int heads, int d,
                         int dtype, void* stream);

/* Block-mean pooling and hybrid block selection [Prism §Blocks: block-level
 * features; hybrid block selection sets each query's sparsity dynamically;
 * configuration examples sparsity 0.75/0.80/0.85/0.93 and CDF threshold 0.20].
 * Reading implemented: qbar/kbar = mean of a block's real tokens (fp64);
 * l_ij = qbar_i . kbar_j / sqrt(d) over the M_v non-empty key blocks (fp64);
 * order by l descending (ties: lower block id first); k = max(1,
 * ceil(M_v (10000 - sparsity_1e4) / 10000)) in integers; m = smallest prefix of
 * that order whose softmax mass reaches tau (>=); the list is the first
 * max(k, m) blocks of the order, emitted in ascending block id.
 *  qp, kp        [heads, Np, d] permuted Q and K (pad slots zero)
 *  sparsity_1e4  skipped fraction x 1e4, 0..9999 (0.85 -> 8500)
 *  tau           CDF threshold, 0 < tau <= 1 (double, so that the threshold
 *                compared against is exactly the caller's value)
 *  counts        [heads, n_blocks] int32 out: list length (0 for an empty query block)
 *  idx           [heads, n_blocks, n_blocks] int32 out: idx[h][i][0..counts) ascending;
 *                entries past counts are left unspecified
 *  pooled_logits [heads, n_blocks, n_blocks] double out, or NULL (debug; -inf
 *                for empty key blocks, rows of empty query blocks unspecified) */
bsa_status bsa_pool_select(const bsa_layout* L, const int32_t* zone_shape, const void* qp,
                           const void* kp, int heads, int d, int dtype, int32_t sparsity_1e4,
                           double tau, int32_t* counts, int32_t* idx, double* pooled_logits,
                           void* ws, size_t ws_bytes, void* stream);

/* The selection half of bsa_pool_select, from block means the caller already
 * has (bsa_permute_pool writes them): same rule, arguments and outputs, with
 *  qbar, kbar  [heads, n_blocks, d] double block means of Q and K (any value
 *              for empty blocks: they are never scored)
 *  ws          workspace of bsa_workspace_size(BSA_CALL_SELECT, ...) bytes */
bsa_status bsa_select(const bsa_layout* L, const int32_t* zone_shape, const double* qbar,
                      const double* kbar, int heads, int d, int32_t sparsity_1e4, double tau,
                      int32_t* counts, int32_t* idx, double* pooled_logits, void* ws,
                      size_t ws_bytes, void* stream);

/* Frame-chunk causal selection [post-training page (gist.science, paper
 * 2604.25427), section 2, stage 4: the bidirectional model is distilled into a
 * causal student that generates frames from its own earlier output through a
 * KV cache, under a causal attention mask]. Reading implemented (the page
 * gives no formula): frames form chunks of frames_per_chunk consecutive
 * frames; a block lies in the chunk of its first frame; query block i sees key
 * block j iff chunk(j) <= chunk(i); bsa_select's rule then runs over each
 * row's visible non-empty key blocks (k from their count V_i:
 * max(1, ceil(V_i (10000 - sparsity_1e4) / 10000))). The lists only name
 * visible blocks, so bsa_attn_fwd / bsa_attn_bwd on them are block-causal as
 * they stand.
 *  frames_per_chunk  >= 1, a multiple of the zone's time extent (the block's in
 *                    fixed mode), so no block spans two chunks (BSA_INVALID_ARG
 *                    otherwise)
 *  pooled_logits     as in bsa_select (not masked)
 *  Other arguments, outputs and workspace as bsa_select. */
bsa_status bsa_select_causal(const bsa_layout* L, const int32_t* zone_shape, const double* qbar,
                             const double* kbar, int heads, int d, int32_t sparsity_1e4,
                             double tau, int frames_per_chunk, int32_t* counts, int32_t* idx,
                             double* pooled_logits, void* ws, size_t ws_bytes, void* stream);

/* Block-sparse attention forward [Prism §Blocks: Prism Block Sparse Attention].
 * For every real query slot n of block i: O[n] = sum over real key slots m of
 * the blocks idx[h][i][0..counts) of softmax_m(Q_n . K_m * scale) V_m, and
 * lse[n] = ln sum_m exp(Q_n . K_m * scale). Non-causal, no dropout.
 *  qp, kp, vp  [heads, Np, d] permuted inputs (pad slots zero)
 *  counts, idx lists from bsa_pool_select (any lists obeying its format work:
 *              ascending, unique, non-empty key blocks only)
 *  scale       softmax scale; 0 selects 1/sqrt(d)
 *  op          [heads, Np, d] out (same dtype); pad query slots get unspecified
 *              finite values; rows of empty query blocks get zeros
 *  lse         [heads, Np] float out (natural log); -inf for rows of empty
 *              query blocks
 *  ws          workspace of bsa_workspace_size(BSA_CALL_ATTN_FWD, ...) bytes (a
 *              per-block table; 0 bytes, ws may be NULL, when that size is 0)
 *  qp, kp, vp and op must be 16-byte aligned (BSA_INVALID_ARG otherwise).
 *  Supported: dtype BSA_BF16 or BSA_F32, d in {64, 128}, B in {64, 128}. Only
 *  bf16 with d = 128 and B = 128 runs on the matrix cores; every other
 *  supported configuration (fp32, d = 64, 64-token blocks) takes a scalar
 *  kernel (one thread per query, K and V staged as fp32 in LDS): a correct
 *  but far slower path, meant for checking, not for speed. */
bsa_status bsa_attn_fwd(const bsa_layout* L, const int32_t* zone_shape, const void* qp,
                        const void* kp, const void* vp, const int32_t* counts,
                        const int32_t* idx, int heads, int d, int dtype, float scale, void* op,
                        float* lse, void* ws, size_t ws_bytes, void* stream);

/* bsa_attn_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * no workspace argument, and the call allocates nothing. The per-block table
 * lives in a static device array of the library (BSA_MAX_BLOCKS x 32 bytes =
 * 128 KiB, enough for every layout the library accepts; BSA_LAYOUT if a layout
 * ever needed more), one per GPU, held until the process ends. Its device
 * address is looked up once per device, on the first call there. Every call on
 * a GPU shares that GPU's array and rewrites the part it uses before reading
 * it; calls that overlap in time on one GPU (concurrent streams, or threads)
 * race on it and must be ordered by the caller. Arguments, outputs and
 * arithmetic are those of bsa_attn_fwd; this is the one call that keeps state
 * (the array and the per-device addresses) across calls. */
bsa_status bsa_attn_fwd_noalloc(const bsa_layout* L, const int32_t* zone_shape, const void* qp,
                                const void* kp, const void* vp, const int32_t* counts,
                                const int32_t* idx, int heads, int d, int dtype, float scale,
                                void* op, float* lse, void* stream);

/* bsa_attn_fwd writing O and lse straight in raster token order (so that the
 * forward path needs no bsa_unpermute of O):
 *  o    [heads, N, d] out, the rows of the real tokens (every one is written)
 *  lse  [heads, N] float out
 *  Same arithmetic and other arguments as bsa_attn_fwd; supported for the
 *  bf16, d = 128, 128-token-block configuration (BSA_UNSUPPORTED otherwise).
 *  The backward takes the permuted O of bsa_attn_fwd. */
bsa_status bsa_attn_fwd_raster(const bsa_layout* L, const int32_t* zone_shape, const void* qp,
                               const void* kp, const void* vp, const int32_t* counts,
                               const int32_t* idx, int heads, int d, int dtype, float scale,
                               void* o, float* lse, void* ws, size_t ws_bytes, void* stream);

/* bsa_attn_fwd_raster reading Q, K and V in raster token order too [Prism
 * §Blocks: attention runs on the tokens regrouped into the zones' blocks;
 * here the regrouping is done by the attention's own tile loads, so the
 * forward path stores no block-ordered copy of Q, K or V]:
 *  q, k, v  [heads, N, d] bf16, the token-order tensors bsa_permute would take
 *  o        [heads, N, d] out, lse [heads, N] float out (as bsa_attn_fwd_raster)
 *  ws       workspace of bsa_workspace_size(BSA_CALL_ATTN_FWD, ...) bytes
 *  Same lists, arithmetic and results as bsa_permute followed by
 *  bsa_attn_fwd_raster, for finite inputs (a pad slot's key and value rows are
 *  read from whatever token sits at its place on the grid, or as zeros past
 *  the last token, and take no weight: the scores of pad keys are masked).
 *  Supported for bf16, d = 128, 128-token blocks, every candidate block shape
 *  of a width that is a multiple of 4, and Np * 256 < 2^31 (BSA_UNSUPPORTED
 *  otherwise: then use bsa_permute + bsa_attn_fwd_raster). q, k, v, o 16-byte
 *  aligned. */
bsa_status bsa_attn_fwd_gather(const bsa_layout* L, const int32_t* zone_shape, const void* q,
                               const void* k, const void* v, const int32_t* counts,
                               const int32_t* idx, int heads, int d, int dtype, float scale,
                               void* o, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Block-sparse attention backward over the forward's lists and lse [Prism
 * §Blocks: Prism Block Sparse Attention is switched on in the training
 * configuration and reported to train 2.5x faster than full attention; Prism
 * §Data ("데이터 준비와 학습 절차", data preparation and training procedure):
 * the whole model is trained with that configuration, so the attention over
 * the selected blocks needs its gradients]. The gradients are those of the
 * forward's function with the lists held fixed (selection is a discrete
 * choice and passes no gradient):
 * D_n = dO_n . O_n; dV_m = sum_n P_nm dO_n; dS_nm = P_nm (dO_n . V_m - D_n);
 * dQ_n = scale sum_m dS_nm K_m; dK_m = scale sum_n dS_nm Q_n; sums over the
 * selected (query, real key) pairs only.
 *  op, lse     forward outputs; dop [heads, Np, d] permuted output gradient
 *              (pad query slots must be zero, as bsa_permute writes them)
 *  dqp, dkp, dvp [heads, Np, d] float32 out, whatever `dtype` is (gradients
 *              are accumulated and returned in fp32); pad slots get zeros.
 *  qp, kp, vp, op, dop must be 16-byte aligned (BSA_INVALID_ARG otherwise).
 *  The key-major (transposed) lists are built in the workspace, with the
 *  order in which the dK/dV pass takes the key blocks (longest list first).
 *  As for the forward, only bf16 with d = 128 and B = 128 runs on the matrix
 *  cores; the other supported configurations take scalar kernels (far
 *  slower). */
bsa_status bsa_attn_bwd(const bsa_layout* L, const int32_t* zone_shape, const void* qp,
                        const void* kp, const void* vp, const void* op, const void* dop,
                        const float* lse, const int32_t* counts, const int32_t* idx,
                        int heads, int d, int dtype, float scale, void* dqp, void* dkp,
                        void* dvp, void* ws, size_t ws_bytes, void* stream);

/* bsa_attn_bwd writing dQ, dK and dV straight in raster token order [Prism
 * §Blocks: attention runs on the tokens regrouped into the zones' blocks, so
 * its gradients are in block order and go back to the latent token order the
 * rest of the model uses; Prism §Data: training runs BSA]:
 *  dq, dk, dv  [heads, N, d] float32 out, the rows of the real tokens (every
 *              one is written; bitwise the rows bsa_unpermute would take from
 *              bsa_attn_bwd's outputs)
 *  Same arithmetic and other arguments as bsa_attn_bwd (the inputs stay in
 *  block order); supported for the bf16, d = 128, 128-token-block
 *  configuration (BSA_UNSUPPORTED otherwise). */
bsa_status bsa_attn_bwd_raster(const bsa_layout* L, const int32_t* zone_shape, const void* qp,
                               const void* kp, const void* vp, const void* op, const void* dop,
                               const float* lse, const int32_t* counts, const int32_t* idx,
                               int heads, int d, int dtype, float scale, void* dq, void* dk,
                               void* dv, void* ws, size_t ws_bytes, void* stream);

/* Audio-to-video cross-attention layer, forward [Prism §Blocks: the zone's
 * block shape uses the feature norm of the audio-to-video cross-attention, in
 * which video tokens attend to the audio tokens]. Reading implemented (the
 * page gives no layer definition): H heads of d = 128, weights in [out, in]
 * layout, no biases:
 *   Q = X Wq^T, K = A Wk^T, V = A Wv^T (D = 128 H columns, head h = columns
 *   128 h .. 128 h + 127), O_h = softmax(Q_h K_h^T / sqrt(128)) V_h over all
 *   audio tokens, lse_h = ln of its denominator, Y = O Wo^T.
 * Products accumulate in fp32; Q, K, V, O and Y are stored as bf16.
 *  n_video   N >= 1 video tokens; n_audio 1..256 audio tokens
 *  C         feature channels, 64..8192, a multiple of 64
 *  heads     1..64; d must be 128 (BSA_UNSUPPORTED otherwise)
 *  x [N, C], a [n_audio, C], wq, wk, wv [D, C], wo [C, D]   bf16, row-major,
 *            16-byte aligned
 *  q [N, D], k [n_audio, D], v [n_audio, D], o [N, D]       bf16 out (the
 *            backward takes them)
 *  lse [heads, N] float out; y [N, C] bf16 out
 *  No workspace. */
bsa_status bsa_xattn_fwd(int n_video, int n_audio, int C, int heads, int d, const void* x,
                         const void* a, const void* wq, const void* wk, const void* wv,
                         const void* wo, void* q, void* k, void* v, void* o, float* lse, void* y,
                         void* stream);

/* [host only] Workspace bytes of bsa_xattn_bwd (0 with the last error set
 * for invalid sizes). */
size_t bsa_xattn_bwd_workspace_size(int n_video, int n_audio, int C, int heads);

/* A2V cross-attention layer, backward of bsa_xattn_fwd (same reading): the
 * gradients of sum(Y * dY),
 *   dO = dY Wo, dWo = dY^T O; per head P = exp(S - lse), dP = dO_h V_h^T,
 *   D = rowsum(dO_h * O_h), dS = P (dP - D), dQ_h = dS K_h / sqrt(128),
 *   dK_h = dS^T Q_h / sqrt(128), dV_h = P^T dO_h;
 *   dX = dQ Wq, dWq = dQ^T X, dA = dK Wk + dV Wv, dWk = dK^T A, dWv = dV^T A.
 * dO, dQ, dK, dV are stored as bf16 in the workspace; products accumulate in
 * fp32; dK, dV are summed over query splits in a fixed order (deterministic).
 *  x, a, wq, wk, wv, wo      as given to bsa_xattn_fwd
 *  q, k, v, o, lse           bsa_xattn_fwd's outputs
 *  dy [N, C] bf16            output gradient
 *  dx [N, C], da [n_audio, C], dwq, dwk, dwv [D, C], dwo [C, D]   float out
 *  ws  workspace of bsa_xattn_bwd_workspace_size(...) bytes, 16-byte aligned
 *  Sizes and alignment as bsa_xattn_fwd. */
bsa_status bsa_xattn_bwd(int n_video, int n_audio, int C, int heads, int d, const void* x,
                         const void* a, const void* wq, const void* wk, const void* wv,
                         const void* wo, const void* q, const void* k, const void* v,
                         const void* o, const float* lse, const void* dy, float* dx, float* da,
                         float* dwq, float* dwk, float* dwv, float* dwo, void* ws,
                         size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H_ */

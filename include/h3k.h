/*
 * h3k — W8A8 DiT block forward for AMD Instinct MI355X (gfx950).
 *
 * C ABI of the library libh3k.so. The operation is the forward pass of one DiT
 * transformer block of the MiniMax-H3 video/audio denoiser, run at every denoising
 * step, as described by the pages:
 *   - "h3-metal: Apple Silicon을 위한 네이티브 MiniMax-H3 추론", section "Int8 양자화"
 *     (native int8 MLP with dynamic activation quantisation and per-output-channel
 *     weight scales; int8 QKV; the QKV and MLP activation quantisers folded into the
 *     preceding gated AdaLN kernel), section "Metal 4 및 TensorOps" (QKV and
 *     attention-output projections routed straight into head-major attention inputs),
 *     and the "속도 및 품질 트레이드오프" table (50 blocks; token reduction pairs
 *     horizontal video tokens in the middle blocks);
 *   - "맥북에서 AI 영상 생성 모델 돌리기 - MiniMax H3 로컬 실행과 30초 애니메이션 만들기",
 *     section "int8 이 뭔가요" (one F32 scale per weight output channel, activations
 *     quantised on the fly with one F32 scale per row);
 *   - "MiniMax-H3在Apple Silicon上的兩種推理實現工程取舍", section 性能上限 (AdaLN gating,
 *     RoPE and quantisation folded into the preceding kernel).
 *
 * Block equations (the pages name the parts; the plainest consistent reading is used):
 *   m = W_ada c = [shift1 | scale1 | gate1 | shift2 | scale2 | gate2]      (6 x d)
 *   h  = LN(x)(1 + scale1) + shift1;     (qa, sa) = quant(h)
 *   [Q|K|V] = (qa Wqkv^T) sa sw;  Q, K <- 3D RoPE;  O = softmax(Q K^T / sqrt(Dh)) V
 *   x1 = x + gate1 * dequant(quant(O) Wo^T)
 *   h2 = LN(x1)(1 + scale2) + shift2;    g = GELU(dequant(quant(h2) Wup^T))
 *   x2 = x1 + gate2 * dequant(quant(g) Wdown^T)
 * LN: LayerNorm without affine, eps from h3k_dims. quant: symmetric per-row int8,
 * s = max|v| / 127 (fp32), q = clamp(rint(v * (127 / max|v|)), -127, 127); a zero row
 * gets s = 0. GELU: exact erf form. RoPE: interleaved pairs (2i, 2i+1); the Dh/2 pairs
 * are split over the token's (t, h, w) grid position: t takes Dh/2 - 2*floor(Dh/6)
 * pairs, h and w floor(Dh/6) each; pair j of an axis with P pairs turns by
 * pos * theta^(-j/P). Tokens are ordered l = (t*Hg + h)*Wg + w.
 *
 * Conventions for every entry point:
 *   - Pointers named as device pointers must be device memory of the current HIP device
 *     (for example torch allocations), 16-byte aligned. The caller owns every buffer;
 *     the library allocates no caller-visible memory and keeps no state between calls
 *     except its profiling records.
 *   - `stream` is a hipStream_t (NULL = the null stream). Calls enqueue work and return
 *     at once; results are ready when the stream reaches them.
 *   - Arguments are validated on the host before any launch. A failed call returns a
 *     negative code, enqueues nothing and sets a thread-local message readable with
 *     h3k_last_error(). NaN and Inf are not checked; they propagate.
 *   - Matrices are row-major. Weights are [N_out, K_in] (K contiguous). bf16 is stored as
 *     its 16-bit pattern (uint16); fp32 as IEEE float.
 *   - Calls on different streams are independent only if their outputs and workspaces
 *     are disjoint.
 *   - Token counts: L (and L / 2 where tokens are paired) must be a multiple of 8, else
 *     H3K_EUNSUPPORTED: the transposed V rows and the attention's key tiles move 8 tokens
 *     per 16-byte access. A grid whose product is not a multiple of 8 is padded by the
 *     caller. Any L that is a multiple of 8 and below 2^24 is supported: partial 256-token
 *     GEMM tiles and partial 64-key attention tiles are masked. (Below 2^24 tokens a head's
 *     K and V^T fit the 32-bit byte range of the attention's buffer loads.)
 */
#ifndef H3K_H
#define H3K_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
enum {
  H3K_OK = 0,
  H3K_EINVAL = -1,       /* null or misaligned pointer, inconsistent sizes           */
  H3K_EUNSUPPORTED = -2, /* valid but unsupported shape (head_dim, d % 256, ...)     */
  H3K_ENOSPC = -3,       /* workspace smaller than h3k_workspace_bytes() asks         */
  H3K_EHIP = -4          /* a HIP runtime call or kernel launch failed               */
};

/* flags for the block and stack calls */
enum {
  H3K_F_BF16_GEMM = 1u,  /* no activation quantisation: bf16 x bf16 GEMMs on the dense
                            bf16 weights wb_* (the pages' BF16 baseline)              */
  H3K_F_FP32_DEBUG = 2u, /* fp32 activations end to end (x_in/x_out fp32), same int8
                            GEMMs; every step between the stored tensors is computed
                            in fp64 and rounded to fp32 once where it is stored: AdaLN
                            modulation, LayerNorm statistics, the GEMM epilogues
                            (dequant, RoPE, GELU, gated residual) and attention
                            (without matrix cores)                                     */
  H3K_F_SYNC = 4u,       /* synchronise the stream and check for errors after every
                            launch (debugging)                                        */
  /* Per-projection precision, for the pages' precision series (BF16 -> int8 MLP -> int8
   * MLP and QKV; "h3-metal: Apple Silicon을 위한 네이티브 MiniMax-H3 추론", section
   * "Int8 양자화"): each flag runs that projection as a bf16 x bf16 GEMM on wb_*, without
   * its activation quantiser. H3K_F_BF16_GEMM is all three. */
  H3K_F_BF16_QKV = 8u,   /* QKV projection                                            */
  H3K_F_BF16_OUT = 16u,  /* attention output projection                               */
  H3K_F_BF16_MLP = 32u,  /* MLP up and down projections                               */
  /* Attention operand precision. By default the QKV epilogue stores Q, K and V as fp16 and
   * attention runs on fp16 matrix-core operands (P rounded to fp16), with O stored as fp16
   * for its int8 quantiser (bf16 when H3K_F_BF16_OUT consumes it). This flag stores Q, K,
   * V, P and O as bf16 instead (the same instruction rate and bytes, 8 significant bits
   * instead of 11). fp16 holds magnitudes up to 65504: an element of Q * log2(e)/sqrt(Dh),
   * K or V beyond that is stored as +-inf and the rows of attention it touches are not
   * finite; such data takes this flag (bf16 has the fp32 range). Not combinable with
   * H3K_F_FP32_DEBUG. */
  H3K_F_ATTN_BF16 = 64u,
  /* h3k_attention only: q carries the base-2 softmax scale (see h3k_attention) */
  H3K_F_Q_BASE2 = 128u
};

/* element types */
enum { H3K_DT_F32 = 0, H3K_DT_BF16 = 1, H3K_DT_F16 = 2 };

typedef struct {
  int32_t d;          /* model width = n_heads * head_dim; multiple of 256            */
  int32_t n_heads;
  int32_t head_dim;   /* 64 or 128                                                     */
  int32_t d_ff;       /* MLP width; multiple of 256                                    */
  int32_t d_cond;     /* conditioning width; multiple of 8, at most 8192              */
  int32_t grid_t, grid_h, grid_w; /* token grid; L must equal their product          */
  float rope_theta;   /* 10000                                                          */
  float ln_eps;       /* 1e-6                                                           */
} h3k_dims;

/* One block's weights: all device pointers. */
typedef struct {
  const uint16_t *w_ada;   /* bf16 [6d, d_cond]: the AdaLN modulation linear layer     */
  const int8_t *w_qkv;     /* int8 [3d, d]: rows Q | K | V; head e owns rows
                              e*Dh..(e+1)*Dh-1 of each part                             */
  const float *s_qkv;      /* fp32 [3d]: per-output-channel scales                      */
  const int8_t *w_o;       /* int8 [d, d]   */
  const float *s_o;        /* fp32 [d]      */
  const int8_t *w_up;      /* int8 [F, d]   */
  const float *s_up;       /* fp32 [F]      */
  const int8_t *w_down;    /* int8 [d, F]   */
  const float *s_down;     /* fp32 [d]      */
  const uint16_t *wb_qkv;  /* bf16 originals, read only for projections a bf16 flag
                              selects (may be NULL otherwise)                         */
  const uint16_t *wb_o;
  const uint16_t *wb_up;
  const uint16_t *wb_down;
  const int8_t *wt_qkv;    /* optional: the same int8 codes in the tiled layout of
                              h3k_tile_weights. When set, that W8A8 projection reads
                              these (a faster kernel) and its row-major w_* may be NULL;
                              results are bit-identical either way                    */
  const int8_t *wt_o;
  const int8_t *wt_up;
  const int8_t *wt_down;
  const uint16_t *wbt_qkv; /* optional: the bf16 originals in the tiled layout (the bytes of
                              each [N, K] bf16 matrix through h3k_tile_weights with
                              k_in = 2K); a bf16 projection reads these when set, and its
                              wb_* may then be NULL; bit-identical results either way   */
  const uint16_t *wbt_o;
  const uint16_t *wbt_up;
  const uint16_t *wbt_down;
} h3k_block_weights;

/* Byte offsets of the intermediates inside a block workspace (for inspection). Arrays
 * use the block's activation type T (bf16, or fp32 under H3K_F_FP32_DEBUG). */
typedef struct {
  size_t m;          /* fp32 [6d] modulation                                          */
  size_t rope;       /* rotation table, fp32 (fp64 with H3K_F_FP32_DEBUG), internal layout */
  size_t s_a, s_o, s_a2, s_g;   /* fp32 [L] per-token scales of the four quantisers     */
  size_t qa, qo, qa2;           /* int8 [L, d]                                          */
  size_t qg;                    /* int8 [L, F]                                          */
  size_t q, k;                  /* A [H, L, Dh] head-major, RoPE applied; A is the
                                   attention operand type: fp16 (bf16 with
                                   H3K_F_ATTN_BF16, fp32 with H3K_F_FP32_DEBUG). On the
                                   16-bit paths q is stored times log2(e)/sqrt(Dh) (the
                                   base-2 softmax scale, applied before its one rounding) */
  size_t vt;                    /* A [H, Dh, L] head-major, transposed                  */
  size_t o;                     /* [L, d] attention output, head e in columns e*Dh ..;
                                   fp16 (bf16 with H3K_F_ATTN_BF16 or H3K_F_BF16_OUT,
                                   fp32 with H3K_F_FP32_DEBUG)                          */
  size_t x1;                    /* T [L, d] residual stream after the attention half    */
  size_t g;                     /* T [L, F] GELU output                                 */
  size_t h, h2;                 /* bf16 [L, d] modulated activations feeding a bf16 QKV /
                                   MLP projection (0 when unused)                       */
  size_t total;                 /* bytes needed (= h3k_workspace_bytes)                */
} h3k_ws_layout;

/* Per-output-channel int8 weight quantisation ("맥북에서 AI 영상 생성 모델 돌리기 - MiniMax H3 로컬 실행과 30초 애니메이션 만들기", section "int8 이 뭔가요": one F32
 * scale per weight output channel; "h3-metal: Apple Silicon을 위한 네이티브 MiniMax-H3 추론", section "Int8 양자화": per-output-channel
 * weight scales) of w [n_out, k_in] (device; bf16 or fp32 per w_dtype):
 * scale_out[n] = max_k |w[n,k]| / 127, q_out[n,k] =
 * clamp(rint(w[n,k] * (127 / max_k |w[n,k]|)), -127, 127), decisions in fp32.
 * q_out int8 [n_out, k_in], scale_out fp32 [n_out] (device). k_in % 8 == 0. */
int h3k_quantize_weights(const void *w, int w_dtype, int64_t n_out, int64_t k_in,
                         int8_t *q_out, float *scale_out, void *stream);

/* Workspace bytes one h3k_block_forward call needs for L tokens under `flags`: room for
 * the intermediates of the block the pages describe (see h3k_block_forward). 0 on invalid
 * dims (the message of h3k_last_error is left as it was). */
size_t h3k_workspace_bytes(const h3k_dims *dm, int64_t L, uint32_t flags);

/* Fills *out with the workspace layout for (dm, L, flags) (the intermediates of the block,
 * see h3k_block_forward). Returns H3K_OK, or H3K_EINVAL / H3K_EUNSUPPORTED for the dims
 * and flags h3k_block_forward would refuse. */
int h3k_workspace_layout(const h3k_dims *dm, int64_t L, uint32_t flags, h3k_ws_layout *out);

/* One DiT block forward: the equations at the top of this file, i.e. the gated AdaLN with
 * the activation quantisers folded in, W8A8 QKV with per-output-channel weight scales and
 * RoPE routed into head-major attention inputs, attention, and the W8A8 out-projection and
 * MLP with gated residuals ("h3-metal: Apple Silicon을 위한 네이티브 MiniMax-H3 추론", sections "Int8 양자화" and "Metal 4 및 TensorOps";
 * "MiniMax-H3在Apple Silicon上的兩種推理實現工程取舍", section 性能上限).
 * x_in, x_out: [L, d] bf16 (fp32 under H3K_F_FP32_DEBUG),
 * device; x_out may alias x_in. cond: fp32 [d_cond] device. w: host pointer to a struct
 * of device pointers. L == grid_t*grid_h*grid_w. ws: device workspace of at least
 * h3k_workspace_bytes(dm, L, flags) bytes; after the call it holds the intermediates at
 * the offsets of h3k_workspace_layout. */
int h3k_block_forward(const void *x_in, void *x_out, const float *cond,
                      const h3k_block_weights *w, const h3k_dims *dm, int64_t L,
                      uint32_t flags, void *ws, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): h3k_block_forward with its workspace in
 * a library-owned scratch array of H3K_NOALLOC_MAX_BYTES per GPU (allocated when the
 * library is loaded, held until the process ends) instead of a caller workspace. The call
 * itself allocates nothing and records no profiling events. Arguments, layouts and errors
 * as h3k_block_forward; H3K_ENOSPC when h3k_workspace_bytes(dm, L, flags) exceeds
 * H3K_NOALLOC_MAX_BYTES (e.g. d = 256 up to L ~ 10000; d = 5120 up to L ~ 500). Every call
 * on one GPU shares that GPU's array and leaves its intermediates there (nothing in it
 * needs clearing between calls: each is written before it is read), so calls that overlap
 * on one GPU (several streams or threads) race; serialise them. */
#define H3K_NOALLOC_MAX_BYTES (64u << 20)
int h3k_block_forward_noalloc(const void *x_in, void *x_out, const float *cond,
                              const h3k_block_weights *w, const h3k_dims *dm, int64_t L,
                              uint32_t flags, void *stream);

/* One block on an explicit token grid ("h3-metal: Apple Silicon을 위한 네이티브 MiniMax-H3 추론", the "속도 및 품질 트레이드오프" table: token
 * reduction pairs horizontal tokens in the middle blocks) (T, Hg, Wg) whose w positions are
 * w * w_pos_scale + w_pos_offset in RoPE; dm's own grid fields are ignored and
 * L = T*Hg*Wg. This is the call the stack makes for its horizontally paired middle
 * blocks (T, Hg, Wg/2 with scale 2 and offset 0.5); h3k_block_forward is the case
 * (dm grid, 1, 0). Other arguments as for h3k_block_forward. */
int h3k_block_forward_grid(const void *x_in, void *x_out, const float *cond,
                           const h3k_block_weights *w, const h3k_dims *dm, int32_t T,
                           int32_t Hg, int32_t Wg, float w_pos_scale, float w_pos_offset,
                           uint32_t flags, void *ws, size_t ws_bytes, void *stream);

/* Multi-head softmax attention without mask ("h3-metal: Apple Silicon을 위한 네이티브
 * MiniMax-H3 추론", section "Metal 4 및 TensorOps": attention over head-major Q/K/V):
 * o[l, e*Dh + j] = sum_k softmax_k(q[e,l,:] . k[e,k,:] * softmax_scale) v[e,k,j].
 * q, k: [H, L, Dh]; v: [H, Dh, L] (transposed, as the QKV projection writes it);
 * o: [L, H*Dh]; all device, all of element type `dtype`:
 *   H3K_DT_F16 / H3K_DT_BF16: matrix-core products on 16-bit operands (P rounded to the
 *     same type), fp32 online softmax with softmax_scale * log2(e) rounded to fp32;
 *   H3K_DT_F32: fp64 arithmetic without matrix cores (the debug path), softmax_scale
 *     taken as given, o rounded to fp32 once.
 * head_dim 64 or 128; L % 8 == 0. flags: H3K_F_SYNC and, for 16-bit dtypes,
 * H3K_F_Q_BASE2: q already holds q * softmax_scale * log2(e) (the block's QKV epilogue
 * stores Q that way, so that scores leave the matrix cores as base-2 exponents), and
 * softmax_scale is not applied again. Errors: H3K_EINVAL (null or misaligned pointers,
 * n_heads or L < 1, softmax_scale <= 0, unknown dtype or flags, H3K_F_Q_BASE2 with
 * H3K_DT_F32), H3K_EUNSUPPORTED (head_dim, L % 8, L >= 2^24, n_heads > 65535). */
int h3k_attention(const void *q, const void *k, const void *v, void *o, int32_t n_heads,
                  int64_t L, int32_t head_dim, double softmax_scale, int dtype,
                  uint32_t flags, void *stream);

/* Workspace bytes for h3k_stack_forward (block workspace plus two reduced-token
 * buffers when tr_begin < tr_end). 0 on invalid dims. */
size_t h3k_stack_workspace_bytes(const h3k_dims *dm, int64_t L, int32_t tr_begin,
                                 int32_t tr_end, uint32_t flags);

/* A stack of n_blocks blocks sharing cond ("h3-metal: Apple Silicon을 위한 네이티브 MiniMax-H3 추론": the DiT runs 50 blocks per denoising
 * step, section "고성능 추론 프리셋"; token reduction pairs horizontal tokens in the middle
 * blocks, the "속도 및 품질 트레이드오프" table); blocks: host array of n_blocks weight structs.
 * Blocks [tr_begin, tr_end) run on horizontally paired tokens: before tr_begin,
 * xr[t,h,j] = (x[t,h,2j] + x[t,h,2j+1]) / 2 on the (T, Hg, Wg/2) grid with w positions
 * 2j + 0.5; after tr_end - 1, x[t,h,2j+s] = x_pre[t,h,2j+s] + (xr_out - xr_in)[t,h,j].
 * tr_begin == tr_end disables pairing; it needs an even grid_w and
 * 0 <= tr_begin <= tr_end <= n_blocks. x_out may alias x_in. */
int h3k_stack_forward(const void *x_in, void *x_out, const float *cond,
                      const h3k_block_weights *blocks, int32_t n_blocks,
                      const h3k_dims *dm, int64_t L, int32_t tr_begin, int32_t tr_end,
                      uint32_t flags, void *ws, size_t ws_bytes, void *stream);

/* ---- a denoising loop around the stack ---- */

/* Workspace bytes for h3k_denoise (the stack's, plus the stack output y in the activation
 * type and fp32 velocity v and core residual r, each [L, d]). */
size_t h3k_denoise_workspace_bytes(const h3k_dims *dm, int64_t L, int32_t tr_begin,
                                   int32_t tr_end, uint32_t flags);

/* `steps` Euler steps of a flow-matching sampler on t_k = 1 - k / steps, k = 0 .. steps, with
 * the speed/quality controls of "h3-metal: Apple Silicon을 위한 네이티브 MiniMax-H3 추론",
 * section "속도 및 품질 트레이드오프" (the pages give the controls, not their formulas; this is
 * the plainest reading, and the stack output stands in for the velocity because the
 * patch embedding and output head are not part of the block stack):
 *   - the stack is the first `layers` blocks (active DiT blocks), token pairing on
 *     [tr_begin, tr_end) of them;
 *   - whole-denoiser reuse: the velocity is evaluated afresh at steps k with k % reuse == 0
 *     and at the last step, and reused in between (20 steps: 11 evaluations for reuse 2, 8
 *     for reuse 3);
 *   - core residual reuse: of those evaluations, every core_reuse-th and the last run the
 *     stack (y = stack(x), cached residual r = y - x, v = y); the others use v = x + r;
 *   - update x <- x + (t_{k+1} - t_k) v, stored in the activation type.
 * x: [L, d] noise in, result out (bf16, or fp32 under H3K_F_FP32_DEBUG); other arguments as
 * h3k_stack_forward. Errors: H3K_EINVAL for steps, reuse or core_reuse < 1, layers outside
 * [1, n_blocks] or a pairing range outside [0, layers]; the stack's errors otherwise. */
int h3k_denoise(void *x, const float *cond, const h3k_block_weights *blocks, int32_t n_blocks,
                const h3k_dims *dm, int64_t L, int32_t steps, int32_t reuse, int32_t core_reuse,
                int32_t layers, int32_t tr_begin, int32_t tr_end, uint32_t flags, void *ws,
                size_t ws_bytes, void *stream);

/* ---- the stack step as a HIP graph ---- */

/* A recorded h3k_stack_forward call: its kernels with these exact arguments (pointers,
 * sizes, flags) as one HIP graph, so that a denoising loop launches a whole 50-block step
 * with one call (launch amortisation; "h3-metal: Apple Silicon을 위한 네이티브 MiniMax-H3
 * 추론" and "MiniMax-H3在Apple Silicon上的兩種推理實現工程取舍", section 性能上限, describe
 * the reference's pre-encoded two-part command buffers). */
typedef struct h3k_graph_s h3k_graph;

/* Records the call on `stream` (a created stream: capture is not possible on the null
 * stream) without running it. Arguments and errors as h3k_stack_forward; H3K_F_SYNC is
 * rejected (H3K_EINVAL). Every launch of the graph reads the buffers as they are then, so
 * the caller updates x_in / cond in place between launches and keeps every buffer alive
 * while the graph exists. On success *graph_out owns a graph (free with
 * h3k_graph_destroy); on error it is NULL. */
int h3k_stack_graph_create(const void *x_in, void *x_out, const float *cond,
                           const h3k_block_weights *blocks, int32_t n_blocks,
                           const h3k_dims *dm, int64_t L, int32_t tr_begin, int32_t tr_end,
                           uint32_t flags, void *ws, size_t ws_bytes, void *stream,
                           h3k_graph **graph_out);
/* Enqueues the recorded step on `stream` (any stream). Launches on one workspace must not
 * overlap. */
int h3k_graph_launch(h3k_graph *graph, void *stream);
/* Frees the graph (NULL is ignored). */
void h3k_graph_destroy(h3k_graph *graph);

/* ---- single steps of the block (the same kernels the block call launches) ---- */

/* The gated AdaLN's modulation ("h3-metal: Apple Silicon을 위한 네이티브 MiniMax-H3 추론", section "Int8 양자화"; "MiniMax-H3在Apple Silicon上的
 * 兩種推理實現工程取舍", section 性能上限: AdaLN gating):
 * m[i] = sum_j w_ada[i, j] * cond[j], fp32 accumulation. w_ada bf16 [n_out, d_cond],
 * cond fp32 [d_cond], m fp32 [n_out]; device. d_cond % 8 == 0, d_cond <= 8192. */
int h3k_adaln_modulation(const uint16_t *w_ada, const float *cond, float *m,
                         int64_t n_out, int32_t d_cond, void *stream);

/* The gated AdaLN with its activation quantiser folded in ("h3-metal: Apple Silicon을 위한 네이티브 MiniMax-H3 추론", section "Int8 양자화"):
 * per row l of x [rows, cols] (x_dtype): h = LN(x_l)(1 + scale) + shift in fp32,
 * then per-row int8 quantisation of h: q_out int8 [rows, cols], s_out fp32 [rows].
 * shift, scale: fp32 [cols]. cols % 256 == 0, cols <= 8192. */
int h3k_ln_modulate_quant(const void *x, int x_dtype, const float *shift,
                          const float *scale, int64_t rows, int32_t cols, float eps,
                          int8_t *q_out, float *s_out, void *stream);

/* Per-row int8 quantisation of x [rows, cols] (x_dtype: fp32, bf16 or fp16) into q_out,
 * s_out, by the rule of h3k_quantize_weights ("맥북에서 AI 영상 생성 모델 돌리기 - MiniMax
 * H3 로컬 실행과 30초 애니메이션 만들기", section "int8 이 뭔가요": one F32 scale per
 * activation row). cols % 8 == 0, cols <= 32768. */
int h3k_row_quantize(const void *x, int x_dtype, int64_t rows, int32_t cols,
                     int8_t *q_out, float *s_out, void *stream);

/* The int8 GEMM of the W8A8 projections ("h3-metal: Apple Silicon을 위한 네이티브 MiniMax-H3 추론", section "Int8 양자화": native int8 MLP and
 * QKV) with a raw epilogue: c[m, n] = sum_k a[m, k] * b[n, k] in
 * int32 (exact). a int8 [M, K], b int8 [N, K], c int32 [M, N]; device. N % 256 == 0,
 * K % 128 == 0, M >= 1. */
int h3k_gemm_i8_i32(const int8_t *a, const int8_t *b, int32_t *c, int64_t M, int64_t N,
                    int64_t K, void *stream);

/* Layout change of int8 weights q [n_out, k_in] (row-major, e.g. from
 * h3k_quantize_weights) into q_tiled (same byte count), the operand order of the block's
 * W8A8 GEMMs: 16 x 64 tiles (16 output channels x 64 bytes of K), tile (nb, kb) at byte
 * 1024 (nb (k_in / 64) + kb), and inside a tile lane l's 16 bytes at 16 l: channel
 * 16 nb + l % 16, bytes 64 kb + 16 (l / 16) .. + 15. A permutation: nothing is computed.
 * bf16 weights [n_out, K] are tiled as their bytes (k_in = 2K). q, q_tiled device, not
 * overlapping; n_out % 16 == 0, k_in % 64 == 0. */
int h3k_tile_weights(const int8_t *q, int64_t n_out, int64_t k_in, int8_t *q_tiled, void *stream);

/* h3k_gemm_i8_i32 with b given in the tiled layout of h3k_tile_weights (the kernel the
 * block uses for tiled weights). Same result, sizes and errors. */
int h3k_gemm_i8_i32_tiled(const int8_t *a, const int8_t *b_tiled, int32_t *c, int64_t M,
                          int64_t N, int64_t K, void *stream);

/* Token reduction ("h3-metal: Apple Silicon을 위한 네이티브 MiniMax-H3 추론", the "속도 및 품질 트레이드오프" table: horizontal video tokens
 * paired in the middle blocks): horizontal pairing of x [T*Hg*Wg, d] (x_dtype) into xr and xr_copy
 * [T*Hg*(Wg/2), d]: xr[t,h,j] = (x[t,h,2j] + x[t,h,2j+1]) / 2 (fp32 add, rounded once). */
int h3k_token_pair(const void *x, void *xr, void *xr_copy, int x_dtype, int32_t T,
                   int32_t Hg, int32_t Wg, int32_t d, void *stream);

/* The end of token reduction (same passage): both members of each pair receive the
 * reduced blocks' update, x[t,h,2j+s] = x_pre[t,h,2j+s] + (xr_out[t,h,j] - xr_in[t,h,j]) for s in {0,1},
 * in place on x_pre (fp32 arithmetic, rounded once). */
int h3k_token_unpair(void *x_pre, const void *xr_out, const void *xr_in, int x_dtype,
                     int32_t T, int32_t Hg, int32_t Wg, int32_t d, void *stream);

/* Thread-local message describing the last failed call on this thread ("" if none).
 * Plumbing of this library (no counterpart on the pages). */
const char *h3k_last_error(void);

/* ---- profiling: per-kernel HIP event timing inside block and stack calls (plumbing of
 * this library, for the per-kernel measurements; no counterpart on the pages) ---- */
enum {
  H3K_K_ADALN = 0, H3K_K_ROPE_TABLE, H3K_K_LN_QUANT, H3K_K_GEMM_QKV, H3K_K_ATTENTION,
  H3K_K_ROWQUANT_O, H3K_K_GEMM_O, H3K_K_GEMM_UP, H3K_K_ROWQUANT_G, H3K_K_GEMM_DOWN,
  H3K_K_TOKEN_PAIR, H3K_K_TOKEN_UNPAIR, H3K_K_COUNT
};
/* While enabled, every kernel the block and stack calls launch is bracketed by two HIP
 * events recorded on the call's stream. Enabling clears earlier records. The records are
 * process-wide and not synchronised: enable, run and read from one thread, with no other
 * thread calling the library meanwhile. */
int h3k_profile_enable(int on);
/* Waits for the recorded events and returns, for kernel kind `kind`, the number of
 * launches recorded and their summed duration in milliseconds. */
int h3k_profile_read(int kind, int64_t *count, double *total_ms);

#ifdef __cplusplus
}
#endif
#endif /* H3K_H */

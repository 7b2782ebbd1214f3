/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE layer forward library, libmoe.so.
 *
 * One MoE layer forward of a dots3-note-style (DeepSeek-V3 lineage) model:
 * sigmoid router with bias-for-selection top-k, dispatch into expert-sorted
 * order, SwiGLU experts as grouped GEMMs, an always-on shared expert, and a
 * weighted combine.
 *
 * Sources (page title, then the section or figure):
 *  [DD] "Xiaohongshu dots3 note Open Source Deep Dive: 280B MoE Multimodal
 *       Model" -- §3.1 Expert Routing Mechanism (Dots3MoELayer.forward),
 *       §3.3 single-layer figure, §8.2 Ascend adaptation figure (FUSED_MC2:
 *       dispatch -> gmm1 -> swiglu -> gmm2 -> combine).
 *  [AA] "dots3-note 架构深度解析：16B 激活参数的 280B MoE 如何实现高效推理" --
 *       «核心架构参数一览» table and «稀疏激活Top-8 路由» section (256 routed + 1
 *       shared experts, top-8, sigmoid scoring, noaux_tc, norm_topk_prob,
 *       hidden 5120, moe_intermediate 1536, BF16/FP8).
 *  [D1] "Transformers 中的 dots.llm1（Dots1）模型" -- «MoE 路由与专家相关字段»
 *       table (n_routed_experts, num_experts_per_tok, n_shared_experts,
 *       n_group, topk_group, norm_topk_prob, routed_scaling_factor,
 *       moe_intermediate_size), «并行策略字段» (packed gate_up_proj,
 *       down_proj, grouped_gemm), and the RMSNorm description (fp32
 *       variance, rsqrt, times the weight; rms_norm_eps 1e-6).
 *
 * Conventions for every entry point:
 *  - All tensor arguments are DEVICE pointers owned by the caller, row-major,
 *    16-byte aligned.  The library never allocates, frees, synchronises or
 *    copies to the host; its only global state is the thread-local text of
 *    the last HIP error (moe_last_error_detail) and the per-device scratch
 *    array of moe_layer_forward_noalloc with its looked-up addresses.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *  - Arguments are validated on the host before anything is enqueued; on an
 *    error nothing is enqueued and no output is touched.  Launch failures
 *    return MOE_ERR_HIP.  Device faults surface at the caller's next sync.
 *  - T == 0 is a valid no-op returning MOE_OK.
 *  - Results are deterministic: no floating-point atomics anywhere.
 *  - Calls on different streams are independent if they use different
 *    outputs and workspaces.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* moe_stream_t; /* hipStream_t */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, misaligned pointer, bad size  */
  MOE_ERR_UNSUPPORTED = -2, /* valid but not supported by this library      */
  MOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required   */
  MOE_ERR_HIP = -4          /* a HIP launch or API call failed              */
} moe_status_t;

typedef enum {
  MOE_F32 = 0,      /* IEEE fp32                                             */
  MOE_BF16 = 1,     /* bfloat16                                              */
  MOE_FP8_E4M3 = 2  /* OCP FP8 E4M3 (bias 7, max 448, no inf), gfx950 native */
} moe_dtype_t;

/* Storage of the expert weight matrices (w_gate_up, w_down, w_sh_gate_up,
 * w_sh_down; never the router weight).  Both hold the same values, only the
 * byte order differs; see moe_pack_expert_weights. */
typedef enum {
  MOE_LAYOUT_ROWS = 0,  /* row-major, as the shapes below state              */
  MOE_LAYOUT_TILED = 1  /* 16-row x 64-byte tiles (moe_pack_expert_weights)  */
} moe_layout_t;

/* Layer shape and options; field names follow the model config fields
 * [AA «核心架构参数一览»; D1 «MoE 路由与专家相关字段»]. */
typedef struct moe_config {
  int32_t T;        /* tokens (batch * sequence, flattened)                 */
  int32_t H;        /* hidden_size; multiple of 128                         */
  int32_t E;        /* n_routed_experts; 1..512                             */
  int32_t S;        /* n_shared_experts; 0..4                               */
  int32_t k;        /* num_experts_per_tok; 1..min(E, 16)                   */
  int32_t I;        /* moe_intermediate_size of a routed expert; mult. of 128;
                       FP8 experts: at least 512, else MOE_ERR_UNSUPPORTED
                       (with fewer channels one e4m3 code of h that rounds
                       the other way at a boundary moves y too much); bf16
                       experts: at most 16384                              */
  int32_t I_shared; /* intermediate size of a shared expert; must equal I   */
  int32_t norm_topk_prob;      /* 1: renormalise the k chosen scores        */
  float routed_scaling_factor; /* multiplies the routing weights            */
  int32_t act_dtype;    /* x, router weight and output: MOE_F32 | MOE_BF16  */
  int32_t expert_dtype; /* expert weights: MOE_F32 (act F32), MOE_BF16 or
                           MOE_FP8_E4M3 (act BF16)                          */
  int32_t n_group;      /* router expert groups; 0 or 1: no grouping.  E must
                           be a multiple, with at most 64 groups [D1]       */
  int32_t topk_group;   /* groups a token may choose from, 1..n_group
                           (ignored without grouping); k <= topk_group *
                           E / n_group                                       */
  int32_t expert_layout; /* moe_layout_t of the expert weights; TILED needs
                           H and I times the expert element size to be
                           multiples of 64 bytes (always so with H and I
                           multiples of 128), else MOE_ERR_UNSUPPORTED       */
} moe_config_t;

/* Weights of one layer (device pointers).
 *  w_router     [E, H]        act_dtype; the gate Linear(H -> E, no bias)
 *                             [DD §3.1; §3.3 "Gate (Linear 5120→256)"]
 *  router_bias  [E]           fp32; added to the sigmoid scores for the
 *                             choice of experts only (noaux_tc [AA])
 *  w_gate_up    [E, 2I, H]    expert_dtype; rows [0, I) gate, [I, 2I) up
 *                             (packed gate_up_proj [D1 «并行策略字段»])
 *  w_down       [E, H, I]     expert_dtype (down_proj)
 *  w_sh_gate_up [S, 2I, H], w_sh_down [S, H, I]: the shared experts.
 *  s_*          fp32 block scales, FP8 only (NULL otherwise): one scale per
 *               128 x 128 block of the matching weight, i.e. s_gate_up
 *               [E, 2I/128, H/128], s_down [E, H/128, I/128], and the same
 *               with S for the shared ones.  Dequantised weight =
 *               e4m3 code * block scale.
 *  w_down_f16, w_sh_down_f16: optional (NULL: not used), bf16 experts only:
 *               fp16 copies of w_down and w_sh_down in the same layout, made
 *               once with moe_convert_bf16_to_f16.  Where h between the two
 *               GEMMs is scaled fp16 (the large-tile path, about 96 or more
 *               rows per expert), the down GEMM multiplies fp16 h by fp16
 *               weights and otherwise converts every bf16 weight fragment in
 *               registers, once per 128-row tile that reads it; with the
 *               copies it reads them instead.  Same conversion, so the same
 *               output bit for bit.  w_sh_down_f16 is required with
 *               w_down_f16 when S > 0; either without w_down_f16, or with
 *               non-bf16 experts: MOE_ERR_INVALID_ARG.  Other paths ignore
 *               them.                                                      */
typedef struct moe_weights {
  const void* w_router;
  const float* router_bias;
  const void* w_gate_up;
  const void* w_down;
  const float* s_gate_up;
  const float* s_down;
  const void* w_sh_gate_up;
  const void* w_sh_down;
  const float* s_sh_gate_up;
  const float* s_sh_down;
  const void* w_down_f16;
  const void* w_sh_down_f16;
} moe_weights_t;

/* Expert weight storage [D1 «并行策略字段»: gate_up_proj and down_proj as
 * stacked per-expert matrices].  No arithmetic: copies `count` row-major
 * [rows, cols] matrices of `dtype` elements from src into dst in the
 * MOE_LAYOUT_TILED order.  Each matrix is cut into 16-row x 64-byte tiles
 * (1 KB); tiles are stored row group by row group, and along the row inside
 * a row group; inside a tile the 16-byte chunks are stored chunk-major
 * (chunk c of the tile's 16 rows, then chunk c + 1).  So byte b of row r of
 * matrix m lands at
 *   m*rows*rb + (r/16)*16*rb + (b/64)*1024 + ((b%64)/16)*256 + (r%16)*16 + b%16,
 * rb = cols * element size.  Matrix m starts at the same byte offset in
 * both layouts, so per-expert pointers and the FP8 block scales are
 * unchanged.  Use: pack w_gate_up with (E, 2I, H), w_down with (E, H, I),
 * and the shared ones with S, then set expert_layout = MOE_LAYOUT_TILED.
 * Every GEMM load instruction (64 lanes x 16 bytes) then reads one whole
 * tile, 1 KB contiguous with lane l at byte 16 l, instead of 16 pieces one
 * weight row apart.
 * src and dst: device, 16-byte aligned, not overlapping, count*rows*rb
 * bytes each.  count >= 0 (0: no-op), rows > 0, cols > 0 and dtype a
 * moe_dtype_t, else MOE_ERR_INVALID_ARG (also for null, misaligned or
 * overlapping buffers); rows not a multiple of 16 or rb not a multiple of
 * 64: MOE_ERR_UNSUPPORTED.  Enqueued on `stream`; dst is complete when the
 * stream reaches that point. */
moe_status_t moe_pack_expert_weights(const void* src, void* dst, int64_t count, int32_t rows,
                                     int32_t cols, int32_t dtype, moe_stream_t stream);

/* Optional fp16 copy of bf16 down weights (moe_weights_t w_down_f16 and
 * w_sh_down_f16).  No page fixes the arithmetic of the expert GEMMs beyond
 * their bf16 weights; this is the conversion the large-tile down GEMM applies
 * to each bf16 weight fragment, moved to load time: each of the n bf16 values
 * of src becomes the fp16 value rounded toward zero (exact for |w| in
 * [2^-14, 65504]; below that the fp16 subnormal toward zero; beyond it
 * +-65504; inf and NaN kept).  Element order is kept, so a tiled src gives
 * a tiled dst.  src and dst: device, 16-byte aligned, n*2 bytes each, not
 * overlapping; n >= 0 (0: no-op) and a multiple of 8, else
 * MOE_ERR_INVALID_ARG.  Enqueued on `stream`. */
moe_status_t moe_convert_bf16_to_f16(const void* src, void* dst, int64_t n, moe_stream_t stream);

/* Human-readable text of a status code (static storage). */
const char* moe_status_string(moe_status_t status);

/* Text of the HIP error behind the most recent MOE_ERR_HIP returned on the
 * calling thread ("" if none).  Diagnostic only; the one piece of state the
 * library keeps, and it is thread-local. */
const char* moe_last_error_detail(void);

/* Library version string, e.g. "moe-gfx950 1.0". */
const char* moe_version(void);

/* Bytes of workspace that moe_layer_forward needs for this config (0 if the
 * config is invalid).  moe_route, moe_dispatch, moe_grouped_ffn and
 * moe_combine accept the same workspace; each needs at most this much. */
size_t moe_workspace_size(const moe_config_t* cfg);

/* The intermediates a layer forward leaves in its workspace, for callers that
 * inspect or reuse them (each step of [DD §3.1] / [DD §8.2 figure]):
 *  MOE_WS_TOPK_IDX   int32 [T, k]      router choice (moe_route semantics)
 *  MOE_WS_TOPK_W     fp32  [T, k]      routing weights
 *  MOE_WS_COUNTS     int32 [E]         rows per expert (when opt_counts is NULL)
 *  MOE_WS_OFFSETS    int32 [E + 1]     exclusive scan of the counts
 *  MOE_WS_PERM       int32 [T*k]       sorted row -> flat (token, slot) index
 *  MOE_WS_INV        int32 [T*k]       flat index -> sorted row
 *  MOE_WS_H          [T*k + S*T, I]    h = SiLU(W_g x) * (W_u x) per sorted row
 *                                      (routed rows first, then shared expert s
 *                                      token t at row T*k + s*T + t): bf16, fp32
 *                                      (MOE_F32 experts) or e4m3 codes (FP8);
 *                                      bf16 experts on the large-tile path:
 *                                      fp16 codes c, h = c * 2^e (MOE_WS_H_EXP)
 *  MOE_WS_H_SCALES   fp32  [T*k + S*T, I/128]  FP8 only: h = code * scale
 *  MOE_WS_H_LO       bf16  [T*k + S*T, I]  bf16 experts on the weight-streaming
 *                                      and mid-size paths only: h - bf16(h),
 *                                      rounded to bf16 (h enters the down GEMM
 *                                      as MOE_WS_H + MOE_WS_H_LO)
 *  MOE_WS_H_EXP      int32 [T*k + S*T, ceil(I/256)]  bf16 experts on the
 *                                      large-tile path only: the exponent e of
 *                                      each row and block of 256 h columns,
 *                                      chosen so that the block's largest |c|
 *                                      lies in [2^14, 2^15) (e = 0 for a block
 *                                      of zeros)
 *  MOE_WS_Y          fp32  [T*k, H]    routed expert outputs, sorted rows;
 *                                      bf16 experts on the large-tile path:
 *                                      fp16 codes, y = c * 2^e (MOE_WS_Y_EXP)
 *  MOE_WS_Y_SHARED   fp32  [S, T, H]   shared expert outputs (fp16 codes as
 *                                      MOE_WS_Y on the large-tile path)
 *  MOE_WS_Y_EXP      int32 [T*k + S*T, ceil(H/256)]  large-tile path only:
 *                                      exponents of y and y_shared per row of
 *                                      the sorted row space and 256 columns,
 *                                      as MOE_WS_H_EXP
 *  MOE_WS_BARRIER    uint32 [2]        moe_layer_forward_fused only: its grid
 *                                      barrier's arrival count, then a status
 *                                      word, 0 after a completed launch and
 *                                      1 if a barrier wait timed out (the
 *                                      outputs are then incomplete)
 * Returns the byte offset of `part` inside the workspace of
 * moe_layer_forward (and of the entry points that share it) for this config,
 * or (size_t)-1 if the config is invalid, `part` unknown, or the config holds
 * no such buffer (e.g. MOE_WS_H_SCALES without FP8).  Contents are valid
 * after the call that writes them, until the next call on that workspace. */
typedef enum {
  MOE_WS_TOPK_IDX = 0, MOE_WS_TOPK_W = 1, MOE_WS_COUNTS = 2, MOE_WS_OFFSETS = 3,
  MOE_WS_PERM = 4, MOE_WS_INV = 5, MOE_WS_H = 6, MOE_WS_H_SCALES = 7, MOE_WS_H_LO = 8,
  MOE_WS_Y = 9, MOE_WS_Y_SHARED = 10, MOE_WS_H_EXP = 11, MOE_WS_BARRIER = 12,
  MOE_WS_Y_EXP = 13
} moe_ws_part_t;
size_t moe_workspace_offset(const moe_config_t* cfg, int32_t part);

/* Router [DD §3.1 steps 1-2; AA «稀疏激活»]: for every token t
 *   l[t,e] = Σ_h x[t,h] * w_router[e,h]      (fp32 accumulate, never bf16)
 *   s = 1 / (1 + exp(-l));   c = s + router_bias   (c used for the choice only)
 *   with n_group > 1 [D1 n_group / topk_group]: the experts form n_group
 *       groups of E / n_group consecutive indices; a group's score is the
 *       sum of its two largest c (its only c if it has one expert); only the
 *       experts of the topk_group groups of largest score (lower group index
 *       first among equal scores) take part in the choice below
 *   topk_idx[t, 0..k) = the k experts of largest c, in decreasing c, the lower
 *                       expert index first among equal c
 *   topk_w[t, j] = s[t, idx_j] / Σ_j' s[t, idx_j'] * routed_scaling_factor
 *                  (without the division when norm_topk_prob == 0)
 * x [T, H] act_dtype; topk_idx [T, k] int32; topk_w [T, k] fp32.
 * tie_counts: NULL, or int32[2] that receives the number of tokens whose
 * k-th and (k+1)-th keys, or topk_group-th and next group scores (index 0),
 * resp. some two consecutive chosen keys (index 1), differ by <= 1e-6 in
 * fp32 -- tokens where another choice or slot order is equally valid at
 * fp32 precision.  Workspace: holds the fp32 logits. */
moe_status_t moe_route(const moe_config_t* cfg, const void* x, const moe_weights_t* w,
                       int32_t* topk_idx, float* topk_w, int32_t* tie_counts,
                       void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* Dispatch [DD §3.1 per-expert mask gather; §8.2 "dispatch"]: group the T*k
 * (token, slot) pairs f = t*k + j by expert e = topk_idx[t, j]:
 *   counts[e]   = #{f : e(f) = e}                         int32 [E]
 *   offsets[e]  = Σ_{e' < e} counts[e'], offsets[E] = T*k  int32 [E+1]
 *   inv[f]      = offsets[e(f)] + #{f' < f : e(f') = e(f)} int32 [T*k]
 *   perm[inv[f]] = f                                       int32 [T*k]
 * i.e. a stable counting sort, bit-exact and deterministic.  topk_idx values
 * must lie in [0, E) (not checked on the device).  Workspace: small. */
moe_status_t moe_dispatch(const moe_config_t* cfg, const int32_t* topk_idx, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* inv, void* workspace,
                          size_t workspace_bytes, moe_stream_t stream);

/* Expert FFNs as grouped GEMMs [D1 «并行策略字段» grouped_gemm; DD §8.2
 * "gmm1 -> swiglu -> gmm2"].  For sorted row p of expert e (offsets[e] <= p <
 * offsets[e+1]) and its token t = perm[p] / k:
 *   h = SiLU(Wg_e x_t) * (Wu_e x_t),  SiLU(z) = z / (1 + exp(-z))
 *   y_sorted[p] = Wd_e h                                  fp32 [T*k, H]
 * and for every shared expert s and token t:
 *   y_shared[s, t] = Wd_s (SiLU(Wg_s x_t) * (Wu_s x_t))   fp32 [S, T, H]
 * fp32 accumulation (SiLU in fp32 with the hardware exponential and
 * reciprocal); between the two GEMMs h is stored as two bf16 terms (h and its
 * residue, ~16 significant bits) where the down GEMM streams its weights
 * (fewer than ~96 rows per expert; MOE_WS_H_LO), and on the MFMA-bound
 * large-tile prefill path as fp16 scaled by a power of two per row and 256
 * columns (11 significant bits; MOE_WS_H_EXP), where the down GEMM takes the
 * bf16 weights as fp16 (exact within fp16's normal range, |w| >= 2^-14;
 * smaller weights keep an absolute error below 2^-25); y stays fp32 so that the layer output is
 * rounded only once, in moe_combine.  FP8: x and h are quantised per token per 128 channels to e4m3
 * with scale amax/448 (fp32, see moe_quantize_fp8) before their GEMM; weights
 * use their block scales.  perm and offsets are moe_dispatch outputs (device).
 * Workspace: h and the tile schedule. */
moe_status_t moe_grouped_ffn(const moe_config_t* cfg, const void* x, const moe_weights_t* w,
                             const int32_t* perm, const int32_t* offsets, void* y_sorted,
                             void* y_shared, void* workspace, size_t workspace_bytes,
                             moe_stream_t stream);

/* The two halves of moe_grouped_ffn, for callers that time or overlap them:
 * gate/up + SwiGLU writes h (returned through the workspace), down reads it.
 * moe_expert_gate_up must run before moe_expert_down on the same workspace. */
moe_status_t moe_expert_gate_up(const moe_config_t* cfg, const void* x, const moe_weights_t* w,
                                const int32_t* perm, const int32_t* offsets, void* workspace,
                                size_t workspace_bytes, moe_stream_t stream);
moe_status_t moe_expert_down(const moe_config_t* cfg, const moe_weights_t* w, void* y_sorted,
                             void* y_shared, void* workspace, size_t workspace_bytes,
                             moe_stream_t stream);

/* Combine [DD §3.1 weighted add; §3.3 "Weighted sum" then shared "add"]:
 *   out[t] = Σ_s y_shared[s, t] + Σ_{j=0}^{k-1} topk_w[t, j] * y_sorted[inv[t*k + j]]
 * y_sorted [T*k, H] and y_shared [S, T, H] are fp32 (moe_grouped_ffn outputs);
 * accumulated in fp32 in exactly this order (s ascending, then j ascending),
 * one rounding to act_dtype.  No atomics.  out [T, H] act_dtype. */
moe_status_t moe_combine(const moe_config_t* cfg, const void* y_sorted, const void* y_shared,
                         const float* topk_w, const int32_t* inv, void* out, moe_stream_t stream);

/* FP8 activation quantisation, the input step of the FP8 expert GEMMs
 * (FP8 precision [AA «核心架构参数一览»]; per-token-per-128-channel scales):
 * for row r and channel c of x [rows, cols] bf16,
 *   scale[r, c/128] = amax over the 128-channel block / 448  (fp32; 1.0 for
 *                     an all-zero block), divided in correctly rounded fp32
 *   q[r, c] = e4m3(x[r, c] / scale[r, c/128]), round to nearest even
 * q [rows, cols] uint8 e4m3 codes; scales [rows, cols/128] fp32.
 * cols must be a multiple of 128; x and q 16-byte aligned. */
moe_status_t moe_quantize_fp8(const void* x_bf16, int32_t rows, int32_t cols, uint8_t* q,
                              float* scales, moe_stream_t stream);

/* The whole layer [DD §3.1 Dots3MoELayer.forward]: route -> dispatch ->
 * grouped gate/up + SwiGLU -> grouped down -> combine, enqueued back to back
 * with no host synchronisation.  out [T, H] act_dtype.
 * opt_counts: NULL or int32[E], receives the per-expert row counts.
 * opt_tie_counts: NULL or int32[2], see moe_route.
 * workspace: at least moe_workspace_size(cfg) bytes, 256-byte aligned. */
moe_status_t moe_layer_forward(const moe_config_t* cfg, const moe_weights_t* w, const void* x,
                               void* out, int32_t* opt_counts, int32_t* opt_tie_counts,
                               void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* The whole layer in ONE launch, for the decode regime: the chain route ->
 * dispatch -> gate/up + SwiGLU -> down -> combine that the Ascend adaptation
 * figure [DD §8.2, FUSED_MC2] runs as one fused operator.  A cooperative
 * persistent grid runs the steps as phases separated by grid barriers.
 * Same arguments, outputs and workspace as moe_layer_forward, and the same
 * results up to the summation order of the router logits (a near-tie can
 * pick the other equally valid expert).  Supported where the layer streams
 * weights: bf16 activations and experts, at most 12 routed rows per expert
 * on average (T*k/E), E a multiple of 16; otherwise MOE_ERR_UNSUPPORTED and
 * nothing is enqueued.  The device must hold the whole grid at once
 * (checked by the cooperative launch; MOE_ERR_HIP if it cannot).  The grid
 * barriers wait a bounded time (moe_fused_set_spin_limit): a launch whose
 * wait runs out stops every block and leaves status 1 in the workspace's
 * MOE_WS_BARRIER word 1, which the caller reads after synchronising the
 * stream (the library never synchronises).  Calls that overlap on one
 * workspace race on that counter. */
moe_status_t moe_layer_forward_fused(const moe_config_t* cfg, const moe_weights_t* w,
                                     const void* x, void* out, int32_t* opt_counts,
                                     int32_t* opt_tie_counts, void* workspace,
                                     size_t workspace_bytes, moe_stream_t stream);

/* Bound of each grid-barrier wait of moe_layer_forward_fused, in polls of
 * the arrival counter (each an atomic load and a short sleep, about a
 * microsecond); 0 gives up at the first poll that finds blocks missing (for
 * tests of that path); polls < 0 restores the default (2^22).  Process-wide,
 * read when a launch is enqueued.  Returns the previous value. */
int64_t moe_fused_set_spin_limit(int64_t polls);

/* RMSNorm of the decoder block [DD §3.3 figure "Residual + RMSNorm"; D1:
 * variance in fp32, rsqrt, times the weight]: for every row t of h [T, H]
 *   out[t, c] = gamma[c] * h[t, c] / sqrt(mean_c' h[t, c']^2 + eps)
 * computed in fp32 (sum of squares in a fixed order) with one rounding to
 * act_dtype.  h, gamma [H] and out are act_dtype; out may not alias h.
 * eps must be finite and >= 0. */
moe_status_t moe_rmsnorm(const moe_config_t* cfg, const void* h, const void* gamma, float eps,
                         void* out, moe_stream_t stream);

/* The MoE half of a decoder block [DD §3.3 figure: "Residual + RMSNorm", MoE
 * FFN layer, "Residual + Output"]:
 *   x = moe_rmsnorm(h)           (stored in act_dtype, the layer's input)
 *   out[t] = h[t] + moe_layer_forward(x)[t]
 * with the residual added inside the combine: h + shared + Σ_j w_j y_j is
 * accumulated in fp32 in that order and rounded to act_dtype once.
 * h, out [T, H] act_dtype (out may not alias h); gamma [H] act_dtype.
 * opt_counts, opt_tie_counts and the workspace as for moe_layer_forward;
 * the workspace also holds x (moe_workspace_size covers it). */
moe_status_t moe_block_forward(const moe_config_t* cfg, const moe_weights_t* w, const void* h,
                               const void* gamma, float eps, void* out, int32_t* opt_counts,
                               int32_t* opt_tie_counts, void* workspace, size_t workspace_bytes,
                               moe_stream_t stream);

/* moe_layer_forward that also records HIP events on `stream` at its stage
 * boundaries, for timing each stage on the stream it runs on:
 *   events[0] before the router      events[4] after the gate/up GEMM
 *   events[1] after the router       events[5] after the down GEMM
 *   events[2] after dispatch         events[6] after the combine
 *   events[3] after the FP8 activation quantisation (same point as [2]
 *             when the experts are not FP8)
 * events: 7 hipEvent_t (passed as void*) created by the caller.  Same
 * results and the same launches as moe_layer_forward. */
moe_status_t moe_layer_forward_timed(const moe_config_t* cfg, const moe_weights_t* w,
                                     const void* x, void* out, int32_t* opt_counts,
                                     int32_t* opt_tie_counts, void* workspace,
                                     size_t workspace_bytes, moe_stream_t stream,
                                     void* const* events);

/* Measurement utility, no step of the layer: reads `bytes` (a multiple of
 * 16) of device memory at src (16-byte aligned) as one streaming pass
 * (non-temporal loads, as the decode GEMMs read their weights) with
 * `blocks` workgroups of 256 threads (1..65536), and writes one folded word
 * per block to sink[0, blocks) so the reads cannot be elided.  Its rate is
 * the read ceiling the weight-streaming (decode) GEMMs are compared with.
 * MOE_ERR_INVALID_ARG on bad arguments; bytes == 0 is a no-op. */
moe_status_t moe_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t blocks,
                             moe_stream_t stream);

/* moe_layer_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments otherwise, same launches
 * and results as moe_layer_forward.  The workspace is a device array inside
 * the library, MOE_NOALLOC_SCRATCH_BYTES (96 MiB) per GPU, held from the
 * library's load on that GPU to the end of the process; configurations
 * whose moe_workspace_size exceeds it return MOE_ERR_UNSUPPORTED and enqueue
 * nothing (at the dots3 shapes -- H 5120, 256 + 1 experts, top-8, I 1536 --
 * up to about 370 tokens).  The first call on a device looks up the array's
 * device address (no allocation).  Every call on one GPU shares the array:
 * calls that overlap in time on one GPU (other streams, other host threads)
 * race and must be serialised by the caller; results of a finished call are
 * in `out`, nothing needs to persist in the array between calls. */
#define MOE_NOALLOC_SCRATCH_BYTES (96u * 1024u * 1024u)
moe_status_t moe_layer_forward_noalloc(const moe_config_t* cfg, const moe_weights_t* w,
                                       const void* x, void* out, int32_t* opt_counts,
                                       int32_t* opt_tie_counts, moe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */

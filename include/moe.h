/*
 * moe.h - C ABI of the MI355X (gfx950) MoE-layer forward library.
 *
 * One DeepSeek-V3-style mixture-of-experts layer, as the Kimi-K2-Thinking-NVFP4
 * walk-through of that architecture describes it (pwwt.cn/news/5781524,
 * section 3 "MoE routing"):
 *   moe_route        - MoEGate.forward: FP32 gate linear, per-expert score
 *                      (sigmoid, or sqrtsoftplus per the DeepSeek-V4-Pro
 *                      overview), + e_score_correction_bias, noaux_tc grouped
 *                      top-k, normalisation x routed_scaling_factor
 *                      (sections 3.1-3.3);
 *   moe_permute      - moe_infer's count + argsort into contiguous per-expert
 *                      blocks, and the gather of the rows (section 3.4);
 *   moe_grouped_ffn  - moe_infer's per-expert gate/up/down + SiLU MLP over each
 *                      block (section 3.4);
 *   moe_combine      - moe_infer's put-back x top-k weight sum, plus the
 *                      always-on shared expert(s) of DeepseekV3MoE.forward
 *                      (section 3.4);
 *   moe_forward      - all of the above in one call;
 *   moe_rmsnorm, moe_forward_residual - the decoder layer around the MoE
 *                      (section 3.5): post_attention_layernorm in front, the
 *                      residual added in the combine;
 *   moe_pack_fp4_scales - weight preparation (once per set of weights, outside
 *                      the layer call): MXFP4 / NVFP4 weight scales into the
 *                      packed layout the routed-expert GEMMs read;
 *   moe_convert_mxfp4_to_fp8 - weight preparation: MXFP4 weights into the
 *                      fp8 recipe's format (DeepSeek-V4-Pro overview, convert.py).
 *
 * Conventions for every entry point
 *   - Every buffer pointer is a DEVICE pointer owned by the caller; the library
 *     never allocates, frees or copies to the host, and never synchronises.
 *     Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) as
 *     kernel launches only (no memset or copy), so a call can be captured into a
 *     HIP graph and replayed; make one call outside the capture first, which
 *     does the library's first-use work (loading the kernels; the no-alloc
 *     entry's scratch lookup).
 *   - Inputs are never written (except an `out` that the caller makes the same
 *     buffer as `resid`).  Outputs are fully overwritten.
 *   - Tensor pointers are 16-byte aligned (rows are read in 16-byte pieces);
 *     moe_rmsnorm and moe_forward_residual check this for their tensors.
 *   - `ws` is caller-owned device scratch of at least moe_workspace_bytes(cfg)
 *     bytes, 256-byte aligned.  Two calls that run at the same time need
 *     distinct workspaces.
 *   - Errors are returned synchronously, before anything is enqueued:
 *     MOE_ERR_INVALID_ARGUMENT (null pointer, bad size, inconsistent groups),
 *     MOE_ERR_UNSUPPORTED (a shape or recipe the kernels do not implement),
 *     MOE_ERR_WORKSPACE_TOO_SMALL.  MOE_ERR_LAUNCH reports a failed kernel
 *     launch.  Faults inside kernels surface at the caller's next
 *     synchronisation.  num_tokens == 0 returns MOE_OK and enqueues nothing.
 *   - Matrices are row-major.  Weights use the [out, in] convention of the
 *     checkpoints (the gate matrix is [E, H], 384 x 7168 in the walk-through).
 *
 * Tensor formats by recipe (x = hidden states [T, H]):
 *   MOE_RECIPE_F32       x, expert and shared weights, y_perm, out: fp32.
 *   MOE_RECIPE_BF16      x, expert and shared weights, y_perm, out: bf16.
 *   MOE_RECIPE_FP8_B128  x bf16; routed weights fp8 e4m3fn (OCP) with one fp32
 *                        scale per 128x128 block; routed-expert activations fp8
 *                        e4m3fn with one fp32 scale per (row, 128 channels),
 *                        scale = amax/448 (block size 128: V4-Pro overview,
 *                        kernel.py act_quant_kernel); shared weights, y_perm,
 *                        out bf16.
 *   MOE_RECIPE_MXFP4     x bf16; routed weights MXFP4 = e2m1 packed two per
 *                        byte (low nibble = even column) with one E8M0 scale
 *                        per 32 along the input dimension; routed-expert
 *                        activations MXFP8 = e4m3fn with one E8M0 scale per
 *                        (row, 32 channels), exponent = least e with
 *                        amax <= 448 * 2^e (MXFP4 weights with MXFP8
 *                        activations: ruibaoantu.com 2.8T articles,
 *                        quantisation section); shared weights, y_perm, out bf16.
 *   MOE_RECIPE_NVFP4     x bf16; routed weights NVFP4 = e2m1 packed two per byte
 *                        (low nibble = even column) with one e4m3fn scale code
 *                        per 16 along the input dimension; routed-expert
 *                        activations NVFP4 per (row, 16 channels) with scale
 *                        e4m3(amax/6) (1 when that rounds to 0) and elements
 *                        e2m1(v/scale), stored as their fp16 values (exact):
 *                        x_perm is fp16 [T*k][H] and x_perm_scale unused (weights
 *                        and input activations in 4 bits with an FP8 scale per
 *                        16: walk-through section 4; shared experts excluded);
 *                        shared weights, y_perm, out bf16.
 *   The gate weight and the correction bias are fp32 in every recipe.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_LAUNCH = 4
} moe_status_t;

typedef enum { MOE_SCORE_SIGMOID = 0, MOE_SCORE_SQRTSOFTPLUS = 1 } moe_score_t;

typedef enum {
  MOE_RECIPE_F32 = 0,
  MOE_RECIPE_BF16 = 1,
  MOE_RECIPE_FP8_B128 = 2,
  MOE_RECIPE_MXFP4 = 3,
  MOE_RECIPE_NVFP4 = 4
} moe_recipe_t;

/* Layer shape and routing hyper-parameters (names follow the config.json keys
 * of the walk-through: num_experts_per_tok = top_k, n_group, topk_group,
 * norm_topk_prob, routed_scaling_factor).  Requirements:
 *   num_tokens >= 0; hidden, intermediate, shared_intermediate > 0;
 *   1 <= top_k <= min(num_experts, 16); num_experts <= 1024;
 *   num_experts % n_group == 0; 1 <= topk_group <= n_group <= 64;
 *   n_group > 1 needs at least 2 experts per group;
 *   topk_group * num_experts / n_group >= top_k;
 *   recipes other than F32 need hidden, intermediate and shared_intermediate
 *   to be multiples of 128, and MXFP4 and NVFP4 need hidden and intermediate
 *   to be multiples of 256; F32 needs multiples of 32;
 *   swiglu_limit finite and >= 0.
 * swiglu_limit (the optional SwiGLU truncation of the DeepSeek-V4-Pro overview,
 * FFN entry; the pages give only its name): when > 0, every SwiGLU (routed and
 * shared experts) computes SiLU(min(g, L)) * clamp(u, -L, L) with L the limit,
 * g = W1 x and u = W3 x. */
typedef struct {
  int32_t num_tokens;            /* T */
  int32_t hidden;                /* H */
  int32_t num_experts;           /* E routed experts */
  int32_t top_k;                 /* k */
  int32_t intermediate;          /* I of one routed expert */
  int32_t num_shared;            /* always-on shared experts, >= 0 */
  int32_t shared_intermediate;   /* I of one shared expert */
  int32_t n_group;               /* expert groups (contiguous ranges) */
  int32_t topk_group;            /* groups kept per token */
  int32_t score_func;            /* moe_score_t */
  int32_t norm_topk_prob;        /* 1: weights normalised to sum 1 before scaling */
  float routed_scaling_factor;   /* 2.827 in the walk-through; route_scale 2.5 in V4-Pro */
  int32_t recipe;                /* moe_recipe_t */
  float swiglu_limit;            /* > 0: SwiGLU clamp, see below; 0: none */
} moe_config_t;

/* One set of experts, expert-major and contiguous.
 *   w13: [n][2*I][H]  rows 0..I-1 are gate_proj, rows I..2I-1 are up_proj
 *        (MXFP4, NVFP4: [n][2*I][H/2] bytes);
 *   w2:  [n][H][I]    down_proj (MXFP4, NVFP4: [n][H][I/2] bytes);
 *   w13_scale, w2_scale: FP8_B128: fp32 [n][2I/128][H/128] and [n][H/128][I/128];
 *                        MXFP4: E8M0 bytes, NVFP4: e4m3fn codes, one per G = 32
 *                        (MXFP4) or 16 (NVFP4) input channels, in the PACKED
 *                        layout that moe_pack_fp4_scales writes from the
 *                        row-major [n*2I][H/G] and [n*H][I/G] arrays;
 *                        other recipes: unused (may be NULL).
 * n = num_experts for routed experts; n = num_shared for the shared experts,
 * whose I is shared_intermediate and which always use the plain (F32 or BF16)
 * format of their recipe. */
typedef struct {
  const void* w13;
  const void* w13_scale;
  const void* w2;
  const void* w2_scale;
} moe_weights_t;

/* Bytes of device scratch every entry point below needs for `cfg`
 * (0 when cfg is invalid). */
size_t moe_workspace_bytes(const moe_config_t* cfg);

/* MoEGate.forward (walk-through sections 3.1-3.3).
 *   x [T][H] (fp32 for F32, else bf16), gate_w [E][H] fp32, bias [E] fp32.
 *   Out: topk_idx [T][k] int32 in selection order (key = fp32(score + bias)
 *   descending, ties to the lower expert index), topk_w [T][k] fp32 = the
 *   unbiased scores of the picks normalised to sum 1 (when norm_topk_prob),
 *   times routed_scaling_factor.
 *   Selection and order are those of the exact gate: logits = the fp32 rounding
 *   of the dot products evaluated with exact products and fp64 accumulation,
 *   scores = fp32 roundings of the fp64 score function.  With fp32 activations,
 *   or bf16 activations and fewer than 512 tokens, the gate is computed that way
 *   (fp64 MFMA) and the weights use those exact scores.  With bf16 activations and
 *   512 tokens or more the logits are screened on the bf16 MFMA pipe (each fp32
 *   gate weight split into two bf16 pieces and a remainder, w = w1 + w2 + w3, exact
 *   products, fp32 sums) within eps = gamma_n |x|_2 (|w1|_2 + |w2|_2) + |x|_2 |w3|_2
 *   of the exact dot product (n = 256 + accumulator groups + 2, gamma_n =
 *   n 2^-24 / (1 - n 2^-24), for sums rounding to within 2^-24 relative; the
 *   router allows twice eps), and every expert whose rank that leaves open is
 *   recomputed exactly; a pick whose rank is never in doubt keeps the score of
 *   its screened logit for its weight, within 0.32 (eps + 2 ulp) + ulp of the
 *   exact score. */
moe_status_t moe_route(const moe_config_t* cfg, const void* x, const float* gate_w,
                       const float* bias, int32_t* topk_idx, float* topk_w,
                       void* ws, size_t ws_bytes, void* stream);

/* moe_infer count + argsort + gather (walk-through section 3.4).
 *   topk_idx [T][k] int32 in [0, E); x [T][H].
 *   Out: expert_offsets [E+1] (exclusive prefix sum of per-expert counts;
 *   expert e owns rows [offsets[e], offsets[e+1])); sorted_pair [T*k]: row p
 *   holds the flat pair f = t*k + j, rows of one expert in increasing f (a
 *   stable sort); pair_pos [T*k]: the row of pair f; x_perm [T*k][H]: row p is
 *   x[sorted_pair[p] / k] in the routed-activation format (F32/BF16 copies;
 *   FP8_B128 and MXFP4: e4m3fn codes) and x_perm_scale its scales (fp32
 *   [T*k][H/128] or E8M0 [T*k][H/32]; NULL allowed for F32/BF16). */
moe_status_t moe_permute(const moe_config_t* cfg, const int32_t* topk_idx, const void* x,
                         int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_pos,
                         void* x_perm, void* x_perm_scale, void* ws, size_t ws_bytes,
                         void* stream);

/* moe_infer per-expert MLP (walk-through section 3.4): for every expert e and
 * row p in its block, y_perm[p] = W2_e (SiLU(W1_e x) * (W3_e x)) (clamped as
 * swiglu_limit says) with x =
 * x_perm[p] (dequantised by its scales).  For FP8_B128 and MXFP4 the SwiGLU
 * output is re-quantised to the activation format before the down projection.
 * fp32 accumulation.  y_perm [T*k][H] (fp32 for F32, else bf16). */
moe_status_t moe_grouped_ffn(const moe_config_t* cfg, const int32_t* expert_offsets,
                             const void* x_perm, const void* x_perm_scale,
                             const moe_weights_t* experts, void* y_perm, void* ws,
                             size_t ws_bytes, void* stream);

/* moe_infer put-back + weighted sum, plus DeepseekV3MoE's shared experts
 * (walk-through section 3.4): out[t] = sum_j topk_w[t][j] * y_perm[pair_pos[t*k+j]]
 * + sum_s SharedMLP_s(x[t]).  The residual is not added (the decoder layer
 * adds it, section 3.5).  `shared` may be NULL when num_shared == 0.
 * out [T][H] (fp32 for F32, else bf16). */
moe_status_t moe_combine(const moe_config_t* cfg, const void* y_perm, const int32_t* pair_pos,
                         const float* topk_w, const void* x, const moe_weights_t* shared,
                         void* out, void* ws, size_t ws_bytes, void* stream);

/* DeepseekV3MoE.forward: route, permute, grouped FFN, combine in one call.
 * topk_idx_out [T][k] and topk_w_out [T][k] are optional copies of the
 * routing (NULL to skip). */
moe_status_t moe_forward(const moe_config_t* cfg, const void* x, const float* gate_w,
                         const float* bias, const moe_weights_t* experts,
                         const moe_weights_t* shared, void* out, int32_t* topk_idx_out,
                         float* topk_w_out, void* ws, size_t ws_bytes, void* stream);

/* moe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation and kernels as moe_forward, with the scratch taken from a static
 * device array the library holds on each GPU it runs on (from the first call on
 * that GPU until the process ends) instead of a caller workspace.  The caller still
 * passes inputs and outputs, as for moe_forward.
 *   - Configurations whose moe_workspace_bytes exceeds
 *     moe_forward_noalloc_scratch_bytes() (128 MiB: the decode shapes, e.g.
 *     T = 128, H = 7168, 384 experts, top-8, I = 2048 needs 68 MiB) return
 *     MOE_ERR_WORKSPACE_TOO_SMALL before anything is enqueued.
 *   - Every call on one GPU uses that GPU's one array: calls that can overlap on a
 *     GPU (other streams, other threads) race and must be serialised by the
 *     caller.  The array keeps the last call's contents; no call relies on it
 *     starting at zero.
 *   - MOE_ERR_LAUNCH also reports a failed lookup of the array's device address. */
moe_status_t moe_forward_noalloc(const moe_config_t* cfg, const void* x, const float* gate_w,
                                 const float* bias, const moe_weights_t* experts,
                                 const moe_weights_t* shared, void* out, int32_t* topk_idx_out,
                                 float* topk_w_out, void* stream);

/* Bytes of moe_forward_noalloc's static scratch array (its size limit). */
size_t moe_forward_noalloc_scratch_bytes(void);

/* post_attention_layernorm (walk-through section 3.5; RMSNorm kept in fp32 in
 * the V4-Pro overview): for each token row t of the residual stream resid [T][H]
 * (fp32 for F32, else bf16),
 *   x[t][i] = act( fp32( (resid[t][i] * r) * norm_w[i] ) ),
 *   r = 1 / sqrt( sum_i resid[t][i]^2 / H + eps ),
 * with the sum, the root and both products in fp64 and act the activation format
 * (fp32, or bf16 rounded to nearest even).  norm_w [H] fp32.  x [T][H] must not
 * overlap resid.  Needs no workspace; eps must be finite and >= 0. */
moe_status_t moe_rmsnorm(const moe_config_t* cfg, const void* resid, const float* norm_w, float eps,
                         void* x, void* stream);

/* The MoE half of a decoder layer (walk-through section 3.5) in one call:
 *   out = resid + DeepseekV3MoE( moe_rmsnorm(resid) ),
 * the residual added in fp32 inside the combine before its single rounding.
 * out may be the same buffer as resid (every element is read before it is
 * written, by the same thread).  The normalised rows live in the workspace. */
moe_status_t moe_forward_residual(const moe_config_t* cfg, const void* resid, const float* norm_w,
                                  float eps, const float* gate_w, const float* bias,
                                  const moe_weights_t* experts, const moe_weights_t* shared,
                                  void* out, int32_t* topk_idx_out, float* topk_w_out, void* ws,
                                  size_t ws_bytes, void* stream);

/* Weight preparation for the MXFP4 and NVFP4 recipes (the e2m1 weights with a
 * scale per 32 or 16 input channels, as the moe_weights_t comment lists them).
 * The routed-expert GEMMs read each weight row's scales 256 input channels at a
 * time for 32 rows at once; in the row-major layout those bytes lie scattered
 * over 32 cache lines that are fetched again for every 256 channels.  The packed
 * layout puts them together:
 *   for each block b of 32 consecutive rows, each s = 0 .. row_len/256 - 1 and
 *   each row r of the block: the R = 256/G scale bytes of row 32b + r for input
 *   channels 256s .. 256s+255, at byte ((b * (row_len/256) + s) * 32 + r) * R.
 * The packed array has the same size as the row-major one.
 *   recipe:  MOE_RECIPE_MXFP4 (G = 32, E8M0 bytes) or MOE_RECIPE_NVFP4 (G = 16,
 *            e4m3fn codes); anything else is MOE_ERR_INVALID_ARGUMENT.
 *   rows:    weight rows of the matrix, all experts stacked (n*2I for w13,
 *            n*H for w2); a multiple of 32, else MOE_ERR_UNSUPPORTED.
 *   row_len: input channels of a row (H for w13, I for w2); a multiple of 256,
 *            else MOE_ERR_UNSUPPORTED.
 *   src:     device, row-major [rows][row_len/G] bytes; dst: device, same size.
 *            Both 16-byte aligned and not overlapping (else
 *            MOE_ERR_INVALID_ARGUMENT); dst is fully overwritten.
 * rows == 0 returns MOE_OK and enqueues nothing. */
moe_status_t moe_pack_fp4_scales(int32_t recipe, int64_t rows, int32_t row_len, const void* src,
                                 void* dst, void* stream);

/* Weight conversion MXFP4 -> MOE_RECIPE_FP8_B128 weights (the DeepSeek-V4-Pro
 * overview, lzwjava.github.io, convert.py entry: FP4 e2m1fn to FP8 e4m3fn without
 * loss, with care for the scales).  Run once per set of weights, outside the
 * layer call, on each matrix (w13 with rows = n*2I, row_len = H; w2 with rows =
 * n*H, row_len = I).
 *   w_fp4:   device, packed e2m1 [rows][row_len/2] (low nibble = even column);
 *   w_e8m0:  device, E8M0 bytes [rows][row_len/32], ROW-MAJOR (the layout before
 *            moe_pack_fp4_scales; bytes 0xFF, E8M0's NaN, are not supported);
 *   w_fp8:   device, out: e4m3fn codes [rows][row_len];
 *   w_fp8_scale: device, out: fp32 [rows/128][row_len/128], one per 128 x 128 block;
 *   inexact_blocks: device int32 or NULL; out: the number of blocks not reproduced
 *            exactly.
 * Block B's scale is 2^(E - 127), E the largest E8M0 byte of B's groups; an element
 * with group byte b and e2m1 value q becomes e4m3(q * 2^(b - E)), rounding to
 * nearest with ties to the even code.  Every e2m1 value is an e4m3 value, so a block
 * whose groups' exponents lie within 8 of E is exact (0.5 * 2^-8 is e4m3's smallest
 * subnormal); others lose the values that fall below that and are counted.
 * rows and row_len must be multiples of 128 (else MOE_ERR_UNSUPPORTED); w_fp4, w_fp8,
 * w_fp8_scale and w_e8m0 16-byte aligned, inexact_blocks 4-byte aligned (else
 * MOE_ERR_INVALID_ARGUMENT).  rows == 0 returns MOE_OK and enqueues nothing. */
moe_status_t moe_convert_mxfp4_to_fp8(int64_t rows, int32_t row_len, const void* w_fp4, const void* w_e8m0,
                                      void* w_fp8, float* w_fp8_scale, int32_t* inexact_blocks, void* stream);

/* Human-readable name of a status code (static storage). */
const char* moe_status_string(moe_status_t status);

/* ------------------------------------------------------------------------
 * Instrumentation: per-kernel timing with HIP events on the launch stream.
 * While enabled, every kernel launch the entry points above make is bracketed
 * by two hipEvents recorded on the caller's stream, tagged by kernel kind.
 * Not thread-safe; meant for benchmarks and profiling runs.
 * ------------------------------------------------------------------------ */
typedef enum {
  MOE_K_GATE = 0,              /* gate logits (fp64 MFMA, or the bf16 screen)          */
  MOE_K_ROUTER,                /* score, bias, grouped top-k, weights                 */
  MOE_K_PERM_HIST,             /* counting sort: per-chunk expert histograms          */
  MOE_K_PERM_SCAN,             /* counting sort: prefix sums, expert offsets          */
  MOE_K_PERM_SCATTER,          /* counting sort: stable row positions                 */
  MOE_K_GATHER,                /* row gather (+ activation quantisation)              */
  MOE_K_TILES,                 /* per-expert row-tile list                            */
  MOE_K_FFN_GATE_UP,           /* routed grouped GEMM gate/up + SwiGLU (+ requant)    */
  MOE_K_FFN_DOWN,              /* routed grouped GEMM down projection                 */
  MOE_K_SHARED_GATE_UP,        /* shared expert(s) gate/up + SwiGLU                   */
  MOE_K_SHARED_DOWN_COMBINE,   /* shared down projection (fp32 recipe: + put-back sum) */
  MOE_K_COMBINE,               /* weighted put-back sum (+ shared-expert rows)        */
  MOE_K_RMSNORM,               /* post_attention_layernorm (moe_rmsnorm, residual form) */
  MOE_K_COUNT
} moe_kernel_tag_t;

/* Start recording; room for max_launches bracketed launches (extra launches are
 * not recorded).  Creates the event pool (no device memory is allocated). */
moe_status_t moe_profile_start(int32_t max_launches);

/* Stop recording: waits for the recorded events, writes per tag the summed
 * milliseconds (ms_out[n_tags]) and launch counts (count_out[n_tags]) for tags
 * < n_tags, destroys the events. */
moe_status_t moe_profile_stop(double* ms_out, int64_t* count_out, int32_t n_tags);

/* Name of a kernel tag (static storage). */
const char* moe_kernel_tag_name(int32_t tag);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */

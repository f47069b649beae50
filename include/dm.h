/* dm.h: C ABI of the MI355X (gfx950) DM0-style dual-expert merged-attention library, libdm.so.
 *
 * What the calls compute (the pages, by title and section):
 *  - "DM0 paper definition vs. Dexbotic code" (dregs-remover.com news 27019), section 1, key
 *    architecture conclusion: in every layer the VLM expert and the action expert each make
 *    their own Q/K/V; these are joined along the sequence axis for one attention and split
 *    back, and each expert applies its own O-projection, residual and MLP.  DM0-base: 28
 *    layers per expert, hidden 2048 (VLM) / 1024 (action), 16 query heads, 8 KV heads, head
 *    dim 128, action dim 32, chunk 50.                                  -> dm_merged_layer
 *  - "DM0.5: High-Performance Embodied VLA and OpenDM Open Source Introduction", section 5.1:
 *    the prefix is encoded once and the VLM's per-layer KV cache is kept so later action
 *    steps do not re-run the VLM.                                        -> dm_prefill_kv
 *  - same page, sections 5.2-5.3: action_in_proj -> action expert over the prefix cache ->
 *    action_out_proj gives the velocity; inference Euler-integrates it from random x_1 over
 *    diffusion_steps (default 10).                                       -> dm_suffix_denoise
 *  - same page, section 6.5: shapes, buffer addresses and the step count are fixed when the
 *    graph is captured at start-up; online the graph is replayed once; a different step count
 *    needs a new capture.                                  -> dm_denoise_plan_* (hipGraph)
 *  - same page, section 6.3: FP8 E4M3 GEMMs for the prefix MLP with scales.
 *                                                -> vlm_mlp_dtype = DM_FP8_E4M3, dm_quantize_fp8_rows
 *
 * Numerics (reading of the pages, which are silent): the residual streams, x and every softmax
 * run in float32; matrix operands are the weight dtype (bf16 or fp32) with fp32 accumulation;
 * intermediates between kernels (Q/K/V, attention output, MLP activation) are stored in the
 * weight dtype; rounding to bf16 is round-to-nearest-even.  RMSNorm eps and RoPE base come
 * from dm_config; RoPE is rotate-half with theta_i = base^(-2i/D); query head h reads KV head
 * h / (Hq/Hkv); prefix token j sits at position j and action token s at P_b + s; the time
 * embedding is sin/cos(t * 10000^(-2i/Ha)) added after action_in_proj; Euler takes
 * x <- x - v(x, t_k)/N with t_k = 1 - k/N.
 *
 * Conventions for every call:
 *  - Pointers are device pointers unless marked (host).  Base pointers must be 16-byte aligned.
 *  - Weights use the [out][in] row-major layout; all layers of an expert are stacked with a
 *    leading layer index (layer stride = one layer's tensor).
 *  - Hidden streams, prefix embeddings and x are float32.  KV caches and weight matrices use
 *    dm_config.dtype.  Norm gains and the action head (w_in, b_in, final_norm, w_out, b_out)
 *    are float32.
 *  - KV cache layout [L][B][Hkv][P_cap][D]: one sample's head is P_cap contiguous rows of D.
 *  - prefix_lens [B] int32 on the device, 1 <= P_b <= P_cap.  The host validates only P_cap.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream), never
 *    synchronize, and never allocate device memory, except dm_ctx_create and
 *    dm_denoise_plan_create.  The caller owns every buffer; `ws` is caller-provided scratch of
 *    at least dm_workspace_bytes() bytes, 256-byte aligned; the library keeps no pointer
 *    after a call returns (a plan keeps the ones it was created with).
 *  - Errors: every call returns a dm_status; arguments are fully validated before any HIP
 *    call; no exception crosses the ABI and nothing aborts.  dm_last_error() gives a
 *    thread-local message for the last failure on the calling thread.
 *  - The library never draws random numbers: x at t = 1 is an input.
 */
#ifndef DM_H
#define DM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DM_OK = 0,
  DM_ERR_INVALID_ARG = -1,   /* null pointer, misaligned pointer, bad enum, non-positive size */
  DM_ERR_SHAPE = -2,         /* sizes inconsistent with the config or outside supported range */
  DM_ERR_UNSUPPORTED = -3,   /* valid request this library does not implement */
  DM_ERR_WORKSPACE = -4,     /* ws too small (see dm_workspace_bytes) */
  DM_ERR_PLAN_MISMATCH = -5, /* launch differs from what the plan captured */
  DM_ERR_HIP = -6            /* a HIP runtime call failed; message in dm_last_error() */
} dm_status;

typedef enum { DM_F32 = 0, DM_BF16 = 1, DM_FP8_E4M3 = 2 } dm_dtype;

typedef enum { DM_OP_PREFILL = 0, DM_OP_MERGED_LAYER = 1, DM_OP_DENOISE = 2 } dm_op;

typedef struct {
  int n_layers;      /* L */
  int vlm_hidden;    /* Hv */
  int act_hidden;    /* Ha */
  int vlm_ffn;       /* Fv */
  int act_ffn;       /* Fa */
  int n_q_heads;     /* Hq */
  int n_kv_heads;    /* Hkv; Hq / Hkv must be 1, 2 or 4 */
  int head_dim;      /* D: 32, 64 or 128 */
  int action_dim;    /* A <= 64 */
  int chunk;         /* S: action tokens per chunk, 1..64 */
  float rms_eps;
  float rope_base;
  dm_dtype dtype;          /* DM_F32 or DM_BF16: weight matrices, KV cache, intermediates */
  dm_dtype vlm_mlp_dtype;  /* equal to dtype, or DM_FP8_E4M3 with dtype DM_BF16 */
} dm_config;

/* One expert, every layer stacked.  H = expert hidden, F = expert FFN, QKV = (Hq+2Hkv)*D. */
typedef struct {
  const float *attn_norm; /* [L][H] */
  const void *w_qkv;      /* [L][QKV][H]: rows of the Hq query heads, then Hkv key heads, then Hkv value heads */
  const void *w_o;        /* [L][H][Hq*D] */
  const float *mlp_norm;  /* [L][H] */
  const void *w_gate;     /* [L][F][H]  (E4M3 codes, one byte each, when the MLP is FP8) */
  const void *w_up;       /* [L][F][H]  (E4M3 codes when FP8) */
  const void *w_down;     /* [L][H][F]  (E4M3 codes when FP8) */
  const float *s_gate;    /* [L][F] per-output-channel dequantisation scales (FP8 only, else NULL) */
  const float *s_up;      /* [L][F] */
  const float *s_down;    /* [L][H] */
} dm_expert_weights;

typedef struct {
  dm_expert_weights body; /* H = Ha, F = Fa, never FP8 */
  const float *w_in;      /* [Ha][A]  action_in_proj */
  const float *b_in;      /* [Ha] */
  const float *final_norm;/* [Ha] */
  const float *w_out;     /* [A][Ha]  action_out_proj */
  const float *b_out;     /* [A] */
} dm_action_weights;

typedef struct dm_ctx dm_ctx;
typedef struct dm_plan dm_plan;

const char *dm_version(void);
const char *dm_last_error(void);

/* Validates cfg and binds the context to HIP device `device`.  Allocates nothing on the device. */
dm_status dm_ctx_create(const dm_config *cfg /* (host) */, int device, dm_ctx **out /* (host) */);
void dm_ctx_destroy(dm_ctx *ctx);

/* Bytes of `ws` the op needs for batch B and padded prefix length P_cap; 0 on bad arguments. */
size_t dm_workspace_bytes(const dm_ctx *ctx, dm_op op, int B, int P_cap);

/* Prefix encoding once (page section 5.1): runs the L VLM-expert layers over prefix_embeds
 * [B][P_cap][Hv] (float32, rows >= P_b ignored) with a bidirectional mask among each sample's
 * P_b tokens, and writes every layer's post-RoPE K and V into k_cache / v_cache
 * [L][B][Hkv][P_cap][D] (rows >= P_b left untouched).  prefix_embeds is not modified.
 * With vlm_mlp_dtype = DM_FP8_E4M3 (page section 6.3) the MLP gate/up/down weights are E4M3
 * codes with per-output-channel scales (see dm_quantize_fp8_rows); each MLP input row
 * (RMSNorm output) and each SwiGLU activation row is quantised per token the same way, and
 * y[m][n] = r_m * s_n * sum_k a_q[m][k] w_q[n][k] accumulates in float32. */
dm_status dm_prefill_kv(dm_ctx *ctx, const dm_expert_weights *vlm /* (host) */,
                        const float *prefix_embeds, const int32_t *prefix_lens, int B, int P_cap,
                        void *k_cache, void *v_cache, void *ws, size_t ws_bytes, void *stream);

/* One merged layer (page 1, section 1) at index `layer` of both experts, in place:
 * h_prefix [B][P_cap][Hv] (rows >= P_b untouched) and h_suffix [B][S][Ha].  Prefix rows attend
 * to the sample's P_b prefix tokens; action rows attend to the P_b prefix tokens and all S
 * action tokens.  k_out / v_out: optional [B][Hkv][P_cap][D] receiving this layer's prefix
 * post-RoPE K/V (both NULL or both set). */
dm_status dm_merged_layer(dm_ctx *ctx, const dm_expert_weights *vlm /* (host) */,
                          const dm_expert_weights *act /* (host) */, int layer,
                          float *h_prefix, float *h_suffix, const int32_t *prefix_lens,
                          int B, int P_cap, void *k_out, void *v_out,
                          void *ws, size_t ws_bytes, void *stream);

/* Action-chunk sampling against a cached prefix (page sections 5.2-5.3): x [B][S][A] float32
 * holds the noise at t = 1 on entry and the action chunk at t = 0 on return, after num_steps
 * Euler steps.  Runs eagerly (kernel launches on `stream`). */
dm_status dm_suffix_denoise(dm_ctx *ctx, const dm_action_weights *aw /* (host) */,
                            const void *k_cache, const void *v_cache, const int32_t *prefix_lens,
                            int B, int P_cap, float *x, int num_steps,
                            void *ws, size_t ws_bytes, void *stream);

/* Same computation captured once as a hipGraph (page section 6.5): every pointer, B, P_cap
 * and num_steps are fixed at capture; prefix_lens and the contents of x and the caches stay
 * device data read at replay.  Capture runs on `stream` and synchronizes it. */
dm_status dm_denoise_plan_create(dm_ctx *ctx, const dm_action_weights *aw /* (host) */,
                                 const void *k_cache, const void *v_cache,
                                 const int32_t *prefix_lens, int B, int P_cap, float *x,
                                 int num_steps, void *ws, size_t ws_bytes, void *stream,
                                 dm_plan **out /* (host) */);
/* Replays the plan once on `stream`; num_steps must equal the captured count
 * (else DM_ERR_PLAN_MISMATCH and nothing is launched). */
dm_status dm_denoise_plan_launch(dm_plan *plan, int num_steps, void *stream);
void dm_denoise_plan_destroy(dm_plan *plan);

/* FP8 E4M3 (OCP e4m3fn) row quantisation (page section 6.3), used for weights (one row per
 * output channel) and, inside dm_prefill_kv, for activations (one row per token):
 * scales[r] = max_c |src[r][c]| / 448 (1 for an all-zero row) and
 * dst[r][c] = e4m3(src[r][c] / scales[r]) rounded to nearest even, saturating at +-448; both
 * divisions are correctly rounded float32.  src [rows][cols] bf16, dst [rows][cols] bytes,
 * scales [rows] float32; src and dst 16-byte aligned.  Asynchronous on `stream`. */
dm_status dm_quantize_fp8_rows(const void *src, uint8_t *dst, float *scales, int rows, int cols,
                               void *stream);

#ifdef __cplusplus
}
#endif
#endif /* DM_H */

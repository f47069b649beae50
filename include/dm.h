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
 *  - prefix_lens [B] int32 on the device, 0 <= P_b <= P_cap (a sample may have no prefix token;
 *    values outside are clamped into that range).  The host validates only P_cap.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream), never
 *    synchronize, and never allocate device memory, except dm_ctx_create,
 *    dm_denoise_plan_create and dm_engine_create (and dm_engine_run synchronizes).  The
 *    caller owns every buffer it passes; `ws` is caller-provided scratch of at least
 *    dm_workspace_bytes() bytes, 256-byte aligned; the library keeps no pointer after a call
 *    returns (a plan or an engine keeps the ones it was created with).
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

typedef enum { DM_OP_PREFILL = 0, DM_OP_MERGED_LAYER = 1, DM_OP_DENOISE = 2, DM_OP_TRAIN = 3 } dm_op;

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
  int flags;               /* DM_FLAG_* bits; 0 for the defaults */
} dm_config;

/* dm_config.flags: run the batch-1 suffix denoise as the multi-kernel sequence even where the
 * single-launch kernel applies (the two agree to rounding; used to compare them). */
#define DM_FLAG_MULTI_KERNEL 1
/* dm_config.flags: the action expert is time-modulated (page "DM0.5: High-Performance Embodied
 * VLA and OpenDM Open Source Introduction", section 5.2: time_mlp_in / time_mlp_out and a time
 * modulator in every layer) instead of taking the additive time embedding; the denoise then
 * needs dm_action_weights.tmod and at most DM_TMOD_MAX_STEPS Euler steps. */
#define DM_FLAG_TIME_MODULATION 2
#define DM_TMOD_MAX_STEPS 16
/* dm_config.flags: Qwen3 per-head QK-norm in both experts (page "DM0 paper definition vs.
 * Dexbotic code", section 1: the experts are Qwen3 stacks): every query and key head vector is
 * RMS-normalised over its D dims with the layer's gain (dm_expert_weights.q_norm / k_norm) before
 * RoPE.  The experts' weights then need q_norm and k_norm. */
#define DM_FLAG_QK_NORM 4

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
  const float *q_norm;    /* [L][D] per-head query norm gain (DM_FLAG_QK_NORM only, else NULL) */
  const float *k_norm;    /* [L][D] per-head key norm gain (DM_FLAG_QK_NORM only, else NULL) */
} dm_expert_weights;

/* Time modulation of the action expert (DM_FLAG_TIME_MODULATION), H = Ha.  Per Euler step with
 * time t: c = w_out silu(w_in tau(t) + b_in) + b_out (tau: the sinusoidal time embedding of width
 * H); layer l's modulator m = w_mod[l] silu(c) + b_mod[l] splits into (scale, shift, gate) of the
 * attention norm, then of the MLP norm; each norm becomes h / rms(h) * (1 + scale) + shift
 * (replacing its learned gain) and its sublayer enters the residual as h += gate * out; the
 * final norm is h / rms(h) * (1 + fscale) + fshift with (fscale, fshift) = w_fmod silu(c) + b_fmod. */
typedef struct {
  const float *w_in;    /* [H][H] time_mlp_in */
  const float *b_in;    /* [H] */
  const float *w_out;   /* [H][H] time_mlp_out */
  const float *b_out;   /* [H] */
  const void *w_mod;    /* [L][6H][H], weight dtype: per layer attention scale, shift, gate, MLP scale, shift, gate */
  const float *b_mod;   /* [L][6H] */
  const void *w_fmod;   /* [2H][H], weight dtype: final-norm scale, shift */
  const float *b_fmod;  /* [2H] */
} dm_time_modulation;

typedef struct {
  dm_expert_weights body; /* H = Ha, F = Fa, never FP8 */
  const float *w_in;      /* [Ha][A]  action_in_proj */
  const float *b_in;      /* [Ha] */
  const float *final_norm;/* [Ha] */
  const float *w_out;     /* [A][Ha]  action_out_proj */
  const float *b_out;     /* [A] */
  const dm_time_modulation *tmod; /* (host) set exactly when the config has DM_FLAG_TIME_MODULATION;
                                     then attn_norm, mlp_norm and final_norm are not read */
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
 * codes with per-output-channel scales (see dm_quantize_fp8_rows); each MLP input row (the
 * gain-scaled residual h * g in bf16; RMSNorm's 1/rms scales the GEMM output) and each SwiGLU
 * activation row (bf16) is quantised per token the same way, and
 * y[m][n] = r_m * s_n * sum_k a_q[m][k] w_q[n][k] accumulates in float32. */
dm_status dm_prefill_kv(dm_ctx *ctx, const dm_expert_weights *vlm /* (host) */,
                        const float *prefix_embeds, const int32_t *prefix_lens, int B, int P_cap,
                        void *k_cache, void *v_cache, void *ws, size_t ws_bytes, void *stream);

/* One merged layer (page 1, section 1) at index `layer` of both experts, in place:
 * h_prefix [B][P_cap][Hv] (rows >= P_b untouched) and h_suffix [B][S][Ha].  Prefix rows attend
 * to the sample's P_b prefix tokens; action rows attend to the P_b prefix tokens and all S
 * action tokens.  k_out / v_out: optional [B][Hkv][P_cap][D] receiving this layer's prefix
 * post-RoPE K/V (both NULL or both set).
 * The two experts share only the prefix K/V, so the action expert's kernels run on a second
 * stream that the context owns (default priority), forked from and joined back into `stream`
 * with events: the call's work is complete when `stream` reaches that point, and it may be
 * captured into a graph on `stream`.  The side stream and its events belong to the context:
 * calls on one context from several host threads at once must be serialised. */
dm_status dm_merged_layer(dm_ctx *ctx, const dm_expert_weights *vlm /* (host) */,
                          const dm_expert_weights *act /* (host) */, int layer,
                          float *h_prefix, float *h_suffix, const int32_t *prefix_lens,
                          int B, int P_cap, void *k_out, void *v_out,
                          void *ws, size_t ws_bytes, void *stream);

/* Action-chunk sampling against a cached prefix (page sections 5.2-5.3): x [B][S][A] float32
 * holds the noise at t = 1 on entry and the action chunk at t = 0 on return, after num_steps
 * Euler steps.  Runs eagerly (kernel launches on `stream`).
 * At B = 1 with the DM0-base action expert (hidden 1024, FFN 3072, 16 query / 8 KV heads of dim
 * 128, bf16, S <= 64, A <= 32, P_cap <= 960) the whole chunk is one kernel launch whose 256
 * workgroups run concurrently and hand results to each other through memory (page section 6.4:
 * at small batch the cost is in per-step launches and temporaries); it needs those 256 CUs to
 * itself.  Should its workgroups fail to meet within about two seconds (another kernel occupying
 * CUs), it gives up and x is filled with NaN.  DM_FLAG_MULTI_KERNEL selects the multi-kernel
 * sequence instead. */
dm_status dm_suffix_denoise(dm_ctx *ctx, const dm_action_weights *aw /* (host) */,
                            const void *k_cache, const void *v_cache, const int32_t *prefix_lens,
                            int B, int P_cap, float *x, int num_steps,
                            void *ws, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): dm_suffix_denoise with its workspace taken from a
 * static device buffer of DM_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs
 * on until the process ends (its address on a device is looked up by dm_ctx_create).  A B and
 * P_cap whose dm_workspace_bytes(DM_OP_DENOISE) exceed it return DM_ERR_WORKSPACE and launch
 * nothing.  Allocates nothing.  All calls on one GPU share that GPU's buffer, which keeps the
 * previous call's contents (what must start at zero is cleared by the call's own kernels): calls
 * that overlap on one GPU (two streams, two threads, or two contexts) race and their results
 * are undefined. */
#define DM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
dm_status dm_suffix_denoise_noalloc(dm_ctx *ctx, const dm_action_weights *aw /* (host) */,
                                    const void *k_cache, const void *v_cache,
                                    const int32_t *prefix_lens, int B, int P_cap, float *x,
                                    int num_steps, void *stream);

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
/* Fixed-contract engine (page "DM0.5: High-Performance Embodied VLA and OpenDM Open Source
 * Introduction", section 6.5: at start-up the computation is captured once over static buffers
 * of fixed shape; online a new observation is copied into those buffers and the graph is
 * replayed once; batch, prompt length, chunk shape and step count are fixed, and another step
 * count needs another capture; section 9.1: model-core latency, the GPU computation alone, is a
 * different figure from request latency, which adds the data movement).
 * An engine owns, on the context's device, the prefix embeddings [B][P_cap][Hv] float32, the
 * prefix lengths [B] int32, x [B][S][A] float32, both KV caches [L][B][Hkv][P_cap][D] and one
 * workspace, and a hipGraph of dm_prefill_kv followed by dm_suffix_denoise over them.  The
 * weights passed at creation must stay valid and unchanged while the engine lives. */
typedef struct dm_engine dm_engine;
/* What every request must match (the engine's "capabilities"). */
typedef struct {
  int batch;       /* B */
  int prefix_cap;  /* P_cap: token slots per sample; each request's P_b lies in 0..P_cap */
  int num_steps;   /* Euler steps captured */
  int chunk;       /* S, from the config */
  int action_dim;  /* A, from the config */
  int vlm_hidden;  /* Hv: floats per prefix embedding row, from the config */
} dm_engine_contract;
/* One request: the shape it claims, and host buffers in and out. */
typedef struct {
  int batch, prefix_cap, num_steps;  /* must equal the contract's */
  const float *prefix_embeds;        /* (host) [B][P_cap][Hv]; rows >= P_b are copied, never read */
  const int32_t *prefix_lens;        /* (host) [B] */
  const float *noise;                /* (host) [B][S][A]: x at t = 1 */
  float *actions;                    /* (host) [B][S][A]: receives the chunk at t = 0 */
} dm_engine_request;
/* Allocates the static buffers (zero-filled), captures the graph for B, P_cap and num_steps
 * (the same ranges as dm_prefill_kv and dm_suffix_denoise) and uploads it; `stream` is
 * synchronised.  Allocates device memory. */
dm_status dm_engine_create(dm_ctx *ctx, const dm_expert_weights *vlm /* (host) */,
                           const dm_action_weights *aw /* (host) */, int B, int P_cap, int num_steps,
                           void *stream, dm_engine **out /* (host) */);
dm_status dm_engine_contract_get(const dm_engine *eng, dm_engine_contract *out /* (host) */);
/* Serves one request: a request whose batch, prefix_cap or num_steps differ from the contract
 * returns DM_ERR_PLAN_MISMATCH, a prefix length outside 0..P_cap DM_ERR_SHAPE, a NULL buffer
 * DM_ERR_INVALID_ARG; a rejected request copies and launches nothing.  Otherwise: the three
 * inputs are copied into the static buffers, the graph is replayed once, the chunk is copied
 * to `actions`, and `stream` is synchronised before the call returns.  Requests on one engine
 * must not overlap. */
dm_status dm_engine_run(dm_engine *eng, const dm_engine_request *req /* (host) */, void *stream);
/* The model-core part alone: one replay over the static buffers as they stand (x is denoised
 * in place, so a second replay starts from the previous chunk).  Asynchronous on `stream`. */
dm_status dm_engine_replay(dm_engine *eng, void *stream);
/* Device addresses of the static input / output buffers (any out pointer may be NULL), for
 * callers whose inputs are already on the device. */
dm_status dm_engine_buffers(const dm_engine *eng, float **prefix_embeds /* (host) */,
                            int32_t **prefix_lens /* (host) */, float **x /* (host) */);
void dm_engine_destroy(dm_engine *eng);

/* Gradients written by dm_train_merged_layer, all float32 and overwritten (not accumulated);
 * shapes are one layer's: the action expert's layer tensors, the action head, and the VLM
 * expert's layer-l attention-norm gain [Hv] and Q/K/V projection [QKV][Hv] (its query rows are
 * zero: in one layer they do not reach the loss) plus the prefix hidden [B][P_cap][Hv] (rows
 * >= P_b zero).  The VLM entries and h_prefix may be NULL with knowledge insulation (then they
 * are zero-filled when set); h_prefix may always be NULL. */
typedef struct {
  float *attn_norm, *w_qkv, *w_o, *mlp_norm, *w_gate, *w_up, *w_down; /* action expert, layer l */
  float *w_in, *b_in, *final_norm, *w_out, *b_out;                    /* action head */
  float *vlm_attn_norm, *vlm_w_qkv;                                   /* VLM expert, layer l */
  float *h_prefix;                                                    /* input gradient of h_prefix */
} dm_train_grads;
/* One flow-matching training step on merged layer `layer` (page "DM0.5: High-Performance
 * Embodied VLA and OpenDM Open Source Introduction", section 5.3: x_t = t eps + (1 - t) a, target
 * u_t = eps - a, loss = mean squared error between the velocity and u_t over the valid action
 * dimensions and time slices only; page "DM0 paper definition vs. Dexbotic code", section 1:
 * knowledge insulation keeps the action expert's gradient out of the VLM, which the public code
 * does not).  Per sample b with time t[b]: the action tokens h0 = x_t W_in^T + b_in + tau(t[b])
 * pass layer `layer` of the action expert, attending to its own tokens and to the prefix keys /
 * values that the VLM expert's layer `layer` makes from h_prefix[b] (rows < P_b; the prefix
 * queries, O-projection and MLP do not reach the action tokens in one layer and are not
 * formed), then the final norm and action_out_proj give v.  *loss (device float) =
 * sum(mask (v - u_t)^2) / sum(mask) over the batch (0 if the mask is empty), and `grads`
 * receives its gradients; with knowledge_insulation != 0 the prefix K/V are constants.
 * h_prefix [B][P_cap][Hv], actions / noise / mask [B][S][A] (mask 0 or 1), t [B]: float32.
 * Arithmetic is float32 (bf16 weights are widened exactly); the model must have neither
 * DM_FLAG_TIME_MODULATION nor DM_FLAG_QK_NORM (else DM_ERR_UNSUPPORTED).  ws: at least
 * dm_workspace_bytes(ctx, DM_OP_TRAIN, B, P_cap) bytes.  Like dm_merged_layer, the call runs its
 * independent parts (the prefix K/V projection, the MLP and O weight gradients, the prefix
 * backward) on the context's side stream, forked from and joined back into `stream`; calls on
 * one context from several host threads at once must be serialised. */
dm_status dm_train_merged_layer(dm_ctx *ctx, const dm_expert_weights *vlm /* (host) */,
                                const dm_action_weights *aw /* (host) */, int layer,
                                const float *h_prefix, const int32_t *prefix_lens, int B, int P_cap,
                                const float *actions, const float *noise, const float *t,
                                const float *mask, int knowledge_insulation, float *loss,
                                const dm_train_grads *grads /* (host) */, void *ws, size_t ws_bytes,
                                void *stream);
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

// Internal launch interface between the C-ABI host layer and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dm {

enum Dt { DT_F32 = 0, DT_BF16 = 1 };

// Rows of a token-major activation matrix belong to samples: row m is token (m % rows_per_b) of
// sample (m / rows_per_b).  Prefix rows are valid while their token index is below the sample's
// prefix length; action rows are always valid.
struct RowMap {
  int rows_per_b;
  const int32_t *lens;  // [B] prefix lengths (device)
  int is_prefix;        // 1: prefix tokens (position = token), 0: action tokens (position = P_b + token)
  int cap;              // P_cap: prefix lengths are clamped to [0, cap]
};

// The hidden stream between sublayers.  h is the fp32 residual stream [M][H].  hg holds
// h * gain of the next RMSNorm rounded to the weight dtype (the next GEMM's operand), and ssq
// the sums of squares of h over every 16-column group, [M][H/16]: the next GEMM scales its
// output rows by 1/sqrt(sum(ssq)/H + eps), which completes RMSNorm(h) W^T.  With ssq NULL the
// operand hg is already normalised (the time-modulated norm) and the rows are not scaled.
struct Hidden {
  float *h;
  void *hg;
  float *ssq;
  int H;
};

// Split-K scratch: fp32 partial sums [k_split][M][N].
struct SplitK {
  int k_split;       // number of K slices (1: no split)
  float *part;
};

// C[M x N] = RMSNorm-scaled A W^T for the fused Q/K/V projection: A = in.hg, rows scaled by
// 1/rms from in.ssq, RoPE on query/key columns, queries token-major [M][Hq*D], keys and values
// head-major [B][Hkv][kv_rows][D].
struct QkvArgs {
  Hidden in; int M; float eps;
  const void *w;                 // [(Hq+2Hkv)*D][H]
  void *q; void *k; void *v;
  int kv_rows;
  RowMap rows;
  const float2 *rope;            // [positions][D/2] (cos, sin)
  int Hq, Hkv, D;
  const float2 *rope_rows = nullptr;  // action rows: [M][D/2] (cos, sin) at position P_b + s
  // Qwen3 per-head QK-norm gains [D] (NULL: none).  When set, the product writes Q and K
  // unrotated and a second launch normalises every query / key head vector, then applies RoPE.
  const float *q_norm = nullptr, *k_norm = nullptr;
};
// out.h += A W^T (times gate[n] when gate is set), then out.hg = (h * next_gain) and out.ssq
// for the next sublayer (next_gain NULL: skip them).  Rows outside RowMap untouched.
// FP8 operands (a and w E4M3 codes): C = a_scale[m] * s_w[n] * (A_q W_q^T); both NULL otherwise.
struct ResidArgs {
  const void *a; int M, K;       // A [M][K]
  const void *w;                 // [H][K]
  Hidden out;
  const float *next_gain;
  RowMap rows;
  const float *a_scale = nullptr, *s_w = nullptr;
  const float *gate = nullptr;   // [H] residual gate of the time-modulated expert
};
// act[M x F] = silu(n Wg^T) * (n Wu^T), n = RMSNorm(h) from in.hg / in.ssq.
// FP8 operands: a8 holds the E4M3 codes of in.hg per row with scales a_scale (so the normalised
// row is a_scale[m] * a8[m] / rms), wg / wu hold E4M3 codes with per-channel scales s_gate / s_up.
struct SwigluArgs {
  Hidden in; int M, F; float eps;
  const void *wg, *wu;           // [F][H] each
  void *act;                     // [M][F]
  RowMap rows;
  const void *a8 = nullptr;
  const float *a_scale = nullptr, *s_gate = nullptr, *s_up = nullptr;
};

// Tile plan of one GEMM launch, chosen by the host.
struct GemmPlan {
  int skinny;   // 1: skinny kernel (M <= 128 in row blocks; K split across waves and workgroups), 0: large-tile or tiled kernel
  int nt;       // skinny: output columns per workgroup (16, 32 or 64); large-tile kernel: 64, 128,
                // 256 or 384 columns per tile; 0: the tiled kernel
  SplitK sk;
  int rt = 4;   // skinny: 16-row tiles per workgroup (4: 64 rows, 2: 32 rows, 1: 16 rows)
  int nw = 4;   // skinny: waves per workgroup (4, or 16 for whole-K residual projections)
  int bm = 128; // big: rows per tile (128; 256 with 256 columns; 64 with 128 columns for a few hundred rows; bf16)
};

void launch_qkv(Dt dt, const QkvArgs &a, const GemmPlan &p, hipStream_t s);
void launch_resid(Dt dt, const ResidArgs &a, const GemmPlan &p, hipStream_t s);
void launch_swiglu(Dt dt, const SwigluArgs &a, const GemmPlan &p, hipStream_t s);
// FP8 variants (large-tile kernel, any M; N a multiple of 128 and K of 128).
void launch_resid_fp8(const ResidArgs &a, hipStream_t s);
void launch_swiglu_fp8(const SwigluArgs &a, hipStream_t s);
// Splits that the skinny kernel supports for K (multiple of 4 waves x one MFMA k-chunk).
int gemm_k_quantum(Dt dt);

// Attention of one query set against [prefix keys ; optional action keys].
struct AttnArgs {
  const void *q; int q_rows_per_b;   // token-major [B*q_rows_per_b][Hq*D]
  int suffix;                        // 1: queries are action tokens (see P_b + S keys)
  const void *kp, *vp; int kp_rows;  // prefix keys/values [B][Hkv][kp_rows][D]
  const void *ks, *vs; int S;        // action keys/values [B][Hkv][S][D] (suffix only)
  const int32_t *lens;
  int B, Hq, Hkv, D;
  int n_chunks, chunk_keys;          // split of the key range (chunk_keys multiple of 32)
  void *out;                         // token-major [B*q_rows_per_b][Hq*D]
  void *part;                        // partial results when n_chunks > 1 (see attn_partial_bytes)
};
size_t attn_partial_bytes(Dt dt, int B, int Hkv, int n_qblocks, int n_chunks, int D);
int attn_qblocks(int q_rows, int Hq, int Hkv);
void launch_attention(Dt dt, const AttnArgs &a, hipStream_t s);

void launch_rope_table(float2 *table, int n_pos, int D, float base, hipStream_t s);
// out[b*S + s][i] = table[min(max(lens[b], 0), cap) + s][i]: the RoPE rows of the action tokens.
void launch_rope_rows(const float2 *table, const int32_t *lens, int cap, int B, int S, int D, float2 *out,
                      hipStream_t s);
// h = src (if src != h), hg = h * gain, ssq per 16 columns: the entry into the first sublayer.
void launch_norm_prep(Dt dt, const float *src, const Hidden &hid, const float *gain, int M, hipStream_t s);
// h = x w_in^T + b_in + tau(t), then hg / ssq for the first layer's attention norm.  gain NULL:
// h = x w_in^T + b_in only (the time-modulated expert: no additive tau, the norm is its own launch).
void launch_embed(Dt dt, const float *x, const float *w_in, const float *b_in, const Hidden &hid,
                  const float *gain, int M, int A, float t, hipStream_t s);
// v = n w_out^T + b_out, x -= v / num_steps, n = RMSNorm(h) * gain, or with fscale set the
// time-modulated n = h / rms(h) * (1 + fscale) + fshift.
void launch_velocity_euler(const float *h, const float *gain, const float *w_out,
                           const float *b_out, float *x, int M, int H, int A, float eps,
                           int num_steps, hipStream_t s, const float *fscale = nullptr,
                           const float *fshift = nullptr);
// Time modulation of the action expert: the per-step tables of a chunk.
// tau[k][i] = sinusoidal time embedding of t_k = 1 - k / num_steps, k < num_steps.
void launch_tau_table(float *tau, int num_steps, int H, hipStream_t s);
// Y[m][n] = sum_k f(X[m][k]) W[n][k] + b[n] for m < M <= 16 (f = SiLU when silu_in, else the
// identity); W [N][K] fp32 or in the weight dtype dt; X, Y fp32.
void launch_rows_gemv(Dt dt, const float *X, int M, int K, const void *W, const float *b, float *Y, int N,
                      bool silu_in, hipStream_t s);
// The time-modulated norm: hg[m][i] = h[m][i] / rms(h[m]) * (1 + scale[i]) + shift[i] in the
// weight dtype (rms over the row, eps as in RMSNorm).
void launch_mod_norm(Dt dt, const float *h, void *hg, const float *scale, const float *shift, int M, int H,
                     float eps, hipStream_t s);
// dst[r][:] = e4m3(src[r][:] / scales[r]), scales[r] = max|src[r][:]| / 448 (1 for a zero row);
// src bf16 [rows][cols].
void launch_fp8_quantize_rows(const void *src, uint8_t *dst, float *scales, int rows, int cols,
                              hipStream_t s);

// ------------------------------------------------------------- training step (train.hip)
// Element strides of a GEMM operand X(row, k) = X[zo*so + zi'*si + row*sm + k*sk] (zi' = zi for
// A, zi / bdiv for B).
struct TOperand {
  long so, si, sm, sk;
};
// C[m][n] = alpha * sum_k A(m, k) B(n, k) + beta * C[m][n] over a zo_n x zi_n batch, fp32 math on
// the matrix cores; C = C + zo*c_so + zi*c_si, rows ldc apart.
struct TGemm {
  int M, N, K;
  TOperand a, b;
  int bdiv;
  float *C;
  long ldc, c_so, c_si;
  int zo_n, zi_n;
  float alpha, beta;
  float *part;         // optional split-K scratch (unbatched products only) of part_floats floats
  size_t part_floats;
  int splits, k_per_split;  // set by launch_tgemm
};
void launch_tgemm(const TGemm &g, Dt ta, const void *A, Dt tb, const void *B, hipStream_t s);
void launch_rms_fwd(const float *x, Dt gt, const void *g, float eps, long rows, int H, const int *lens, int rows_per_b,
                    float *y, float *rstd, hipStream_t s);
void launch_rms_bwd(const float *x, Dt gt, const void *g, const float *dy, const float *rstd, const float *add, long rows,
                    int H, float *out, hipStream_t s);
// part: colsum_part_floats(M, N) floats of scratch
void launch_colsum(const float *dy, const float *x, const float *rstd, int M, int N, float *out, float *part,
                   hipStream_t s);
size_t colsum_part_floats(int M, int N);
void launch_rope_rows(float *p, long rows, int rows_per_b, int ld, int col0, int heads, int D, double base,
                      const int *lens, bool after_prefix, float sign, hipStream_t s);
void launch_gather_kv(const float *kvp, const float *qkv, const int *lens, int B, int P_cap, int S, int Hq, int Hkv,
                      int D, float *K, float *V, hipStream_t s);
void launch_scatter_kv(const float *dK, const float *dV, const int *lens, int B, int P_cap, int S, int Hq, int Hkv,
                       int D, float *dqkv, float *dkvp, hipStream_t s);
void launch_softmax_rows(float *sc, const int *lens, int B, int Hq, int S, int P_cap, hipStream_t s);
void launch_softmax_bwd(const float *p, float *dp, long rows, int T, float scale, hipStream_t s);
void launch_fm_embed(const float *a, const float *eps, const float *t, const float *w_in, const float *b_in, int B, int S,
                     int A, int H, float time_base, float *x, float *u, float *h0, hipStream_t s);
void launch_copy_bias(const float *src, const float *bias, long M, int N, float *dst, hipStream_t s);
void launch_fill(float *p, long n, float v, hipStream_t s);
void launch_swiglu_fwd(const float *gt, const float *up, long n, float *act, hipStream_t s);
void launch_swiglu_bwd(const float *gt, const float *up, const float *dact, long n, float *dgt, float *dup, hipStream_t s);
void launch_fm_loss(const float *v, const float *u, const float *mask, long n, float *loss, float *dv, hipStream_t s);

// Single-launch batch-1 suffix denoise (persist.hip): the DM0-base action expert (hidden 1024,
// FFN 3072, 16 query / 8 KV heads of dim 128, bf16) at batch 1, S <= 64 action tokens,
// action dim <= 32 (multiple of 4), P_cap <= 960, at most 28 layers.
struct PersistLaunch {
  const void *w_qkv, *w_o, *w_gate, *w_up, *w_down;
  const float *attn_norm, *mlp_norm, *w_in, *b_in, *final_norm, *w_out, *b_out;
  const void *k_cache, *v_cache;
  const int32_t *lens;
  float *x;
  int L, S, A, P_cap, steps;
  float eps, rope_base;
  void *ws;  // persist_ws_bytes(S, A), 256-byte aligned
};
bool persist_supported(int L, int H, int F, int Hq, int Hkv, int D, int S, int A, int B, int P_cap, bool bf16_dtype);
size_t persist_ws_bytes(int S, int A);
// hipSuccess when the device can hold all 256 workgroups at once
hipError_t persist_check_device(int device);
hipError_t launch_denoise_persistent(const PersistLaunch &p, hipStream_t s);

}  // namespace dm

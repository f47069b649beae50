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
  int cap;              // P_cap: prefix lengths are clamped to it
};

// C[M x N] = A[M x K] * W^T for the fused Q/K/V projection: RoPE on the query and key columns,
// queries stored token-major [M][Hq*D], keys and values head-major [B][Hkv][kv_rows][D].
struct QkvArgs {
  const void *a; int M, K;
  const void *w;                 // [(Hq+2Hkv)*D][K]
  void *q; void *k; void *v;
  int kv_rows;                   // rows per (sample, kv head) in k/v
  RowMap rows;
  const float2 *rope;            // [positions][D/2] (cos, sin)
  int Hq, Hkv, D;
};
// h[M x N] += A[M x K] * W^T (float32 residual stream), rows outside RowMap untouched.
struct ResidArgs {
  const void *a; int M, K, N;
  const void *w;                 // [N][K]
  float *h;                      // [M][N]
  RowMap rows;
};
// act[M x F] = silu(A Wg^T) * (A Wu^T)
struct SwigluArgs {
  const void *a; int M, K, F;
  const void *wg, *wu;           // [F][K] each
  void *act;                     // [M][F]
  RowMap rows;
};

void launch_qkv(Dt dt, const QkvArgs &a, hipStream_t s);
void launch_resid(Dt dt, const ResidArgs &a, hipStream_t s);
void launch_swiglu(Dt dt, const SwigluArgs &a, hipStream_t s);

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
  float *part;                       // partial results when n_chunks > 1
};
size_t attn_partial_bytes(int B, int Hkv, int n_qblocks, int n_chunks, int D);
int attn_qblocks(int q_rows, int Hq, int Hkv);
void launch_attention(Dt dt, const AttnArgs &a, hipStream_t s);

void launch_rope_table(float2 *table, int n_pos, int D, float base, hipStream_t s);
void launch_rmsnorm(Dt dt, const float *h, const float *gain, void *out, int M, int H, float eps,
                    hipStream_t s);
void launch_embed(const float *x, const float *w_in, const float *b_in, float *h, int M, int A,
                  int H, float t, hipStream_t s);
void launch_velocity_euler(const float *h, const float *gain, const float *w_out,
                           const float *b_out, float *x, int M, int H, int A, float eps,
                           int num_steps, hipStream_t s);
void launch_copy_f32(const float *src, float *dst, size_t n, hipStream_t s);
void launch_fp8_quantize_rows(const void *src, uint8_t *dst, float *scales, int rows, int cols,
                              hipStream_t s);

}  // namespace dm

// Small kernels of the path: RoPE table, entry into the first sublayer (h*gain and sums of
// squares), action_in_proj + time embedding, final norm + action_out_proj + Euler update, FP8
// E4M3 row quantisation, and the time-modulated expert's pieces (the chunk's sinusoid table,
// a rows-times-matrix GEMV for its time MLP and modulators, the modulated RMSNorm).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dm {

// (cos, sin) of pos * base^(-2i/D) for every position and pair index, computed in double
// precision and rounded to float: rotate-half RoPE of the Qwen3 experts (page "DM0 paper
// definition vs. Dexbotic code", section 1 names Qwen3).
__global__ void rope_table_kernel(float2 *table, int n_pos, int D, double base) {
  const int half = D / 2;
  const long n = (long)n_pos * half;
  for (long idx = blockIdx.x * (long)blockDim.x + threadIdx.x; idx < n; idx += (long)gridDim.x * blockDim.x) {
    const int pos = (int)(idx / half), i = (int)(idx % half);
    const double theta = pow(base, -2.0 * i / D);
    const double ang = (double)pos * theta;
    table[idx] = make_float2((float)cos(ang), (float)sin(ang));
  }
}
void launch_rope_table(float2 *table, int n_pos, int D, float base, hipStream_t s) {
  const long n = (long)n_pos * (D / 2);
  const int blocks = (int)((n + 255) / 256);
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks < 1024 ? blocks : 1024), dim3(256), 0, s, table, n_pos, D,
                     (double)base);
}

__global__ void rope_rows_kernel(const float2 *__restrict__ table, const int32_t *__restrict__ lens, int cap, int S,
                                 int half, int n, float2 *__restrict__ out) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int i = idx % half, row = idx / half, b = row / S, s = row - b * S;
  const int pos = max(0, min(lens[b], cap)) + s;
  out[idx] = table[(size_t)pos * half + i];
}
void launch_rope_rows(const float2 *table, const int32_t *lens, int cap, int B, int S, int D, float2 *out,
                      hipStream_t s) {
  const int n = B * S * (D / 2);
  hipLaunchKernelGGL(rope_rows_kernel, dim3((n + 255) / 256), dim3(256), 0, s, table, lens, cap, S, D / 2, n, out);
}

// Writes 8 consecutive columns c0..c0+7 of row m: h (if a source is given), hg = h*gain and,
// with the neighbouring lane (c0 ^ 8), the sum of squares of the 16-column group.
template <typename T>
__device__ __forceinline__ void write_hidden8(const Hidden &hid, const float *gain, int m, int c0, const float *v,
                                              bool write_h) {
  float *hr = hid.h + (size_t)m * hid.H + c0;
  T *gr = (T *)hid.hg + (size_t)m * hid.H + c0;
  float sq = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (write_h) hr[e] = v[e];
    gr[e] = from_f32<T>(v[e] * gain[c0 + e]);
    sq += v[e] * v[e];
  }
  sq += dpp<DPP_XOR1>(sq);
  if ((c0 & 15) == 0) hid.ssq[(size_t)m * (hid.H >> 4) + (c0 >> 4)] = sq;
}

// Entry into the first sublayer of a stack: h = src (src may be h itself), hg = h*gain,
// per-16-column sums of squares.  One workgroup per row, 8 columns per thread.
template <typename T>
__global__ __launch_bounds__(256) void norm_prep_kernel(const float *__restrict__ src, Hidden hid, const float *gain) {
  const int m = blockIdx.x;
  const bool copy = src != hid.h;
  for (int c0 = threadIdx.x * 8; c0 < hid.H; c0 += 256 * 8) {
    float v[8];
    const float4 *p = reinterpret_cast<const float4 *>(src + (size_t)m * hid.H + c0);
    const float4 x0 = p[0], x1 = p[1];
    v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w; v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
    write_hidden8<T>(hid, gain, m, c0, v, copy);
  }
}
void launch_norm_prep(Dt dt, const float *src, const Hidden &hid, const float *gain, int M, hipStream_t s) {
  if (dt == DT_BF16)
    hipLaunchKernelGGL(norm_prep_kernel<bf16>, dim3(M), dim3(256), 0, s, src, hid, gain);
  else
    hipLaunchKernelGGL(norm_prep_kernel<float>, dim3(M), dim3(256), 0, s, src, hid, gain);
}

// Page "DM0.5: High-Performance Embodied VLA ...", section 5.2: action_in_proj lifts each
// action vector to the expert width; the flow time enters as sin/cos(t * 10000^(-2i/H)) added
// to every action token: h[m][i] = sum_a x[m][a] w_in[i][a] + b_in[i] + tau_i(t).
// Also writes hg / sums of squares for the first layer's attention norm.  Thread = column i
// (its w_in row loaded once, all loads in flight), workgroup = 256 columns x 8 action tokens.
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const float *__restrict__ x, const float *__restrict__ w_in,
                                                    const float *__restrict__ b_in, Hidden hid,
                                                    const float *__restrict__ gain, int M, int A, float t) {
  constexpr int R = 8;
  __shared__ float xs[R * 64];
  const int H = hid.H, half = H / 2;
  const int m0 = blockIdx.x * R;
  const int i_raw = blockIdx.y * 256 + threadIdx.x;
  const bool col_ok = i_raw < H;  // H is a multiple of 16: whole 16-lane groups agree
  const int i = col_ok ? i_raw : H - 1;
  for (int j = threadIdx.x; j < R * A; j += 256) xs[j] = (m0 + j / A) < M ? x[(size_t)m0 * A + j] : 0.f;
  float4 w4[16];
  const float4 *wr = reinterpret_cast<const float4 *>(w_in + (size_t)i * A);
  const int nw4 = A / 4;
#pragma unroll
  for (int j = 0; j < 16; ++j) w4[j] = wr[min(j, nw4 - 1)];  // unconditional: loads stay in flight
  const float bias = b_in[i], gn = gain ? gain[i] : 0.f;
  // tau in float32: t * omega lies in [0, 1], where sinf / cosf / exp2f are within a few ulp
  // (the double-precision versions added about 1 us to the launch at batch 1)
  const int j = i < half ? i : i - half;
  const float w = exp2f(-2.0f * (float)j / (float)H * 13.287712379549449f);  // 10000^(-2j/H)
  const float tau = gain ? (i < half ? sinf(t * w) : cosf(t * w)) : 0.f;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int m = m0 + r;
    float acc = 0.f;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj)
      if (4 * jj < A) {
        const float *xr = xs + r * A + 4 * jj;
        acc += w4[jj].x * xr[0] + w4[jj].y * xr[1] + w4[jj].z * xr[2] + w4[jj].w * xr[3];
      }
    const float v = acc + bias + tau;
    const float sq = sum16(v * v);
    if (m < M && col_ok) {
      hid.h[(size_t)m * H + i] = v;
      if (gain) {
        ((T *)hid.hg)[(size_t)m * H + i] = from_f32<T>(v * gn);
        if ((i & 15) == 0) hid.ssq[(size_t)m * (H >> 4) + (i >> 4)] = sq;
      }
    }
  }
}
void launch_embed(Dt dt, const float *x, const float *w_in, const float *b_in, const Hidden &hid, const float *gain,
                  int M, int A, float t, hipStream_t s) {
  dim3 grid((M + 7) / 8, (hid.H + 255) / 256);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(embed_kernel<bf16>, grid, dim3(256), 0, s, x, w_in, b_in, hid, gain, M, A, t);
  else
    hipLaunchKernelGGL(embed_kernel<float>, grid, dim3(256), 0, s, x, w_in, b_in, hid, gain, M, A, t);
}


// Page "DM0.5: High-Performance Embodied VLA ...", sections 5.2-5.3: action_out_proj gives the
// velocity and one explicit Euler step moves x toward t = 0:
//   v = RMSNorm(h; gain) w_out^T + b_out ;  x <- x - v / N.
// One workgroup per action token; thread t owns columns 4t.. of every 1024-column block and
// issues its w_out loads 16 outputs at a time, then partial sums reduce across the workgroup.
__global__ __launch_bounds__(256) void velocity_euler_kernel(const float *__restrict__ h, const float *__restrict__ gain,
                                                             const float *__restrict__ w_out,
                                                             const float *__restrict__ b_out, float *__restrict__ x,
                                                             int H, int A, float eps, float inv_steps,
                                                             const float *__restrict__ fscale,
                                                             const float *__restrict__ fshift) {
  __shared__ float red[4][64];
  __shared__ float red1[4];
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float4 hv[4], gv[4], sv[4];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // unconditional loads (clamped column) stay in flight together
    const int c = min(4 * tid + 1024 * j, H - 4);
    hv[j] = *reinterpret_cast<const float4 *>(h + (size_t)m * H + c);
    if (fscale) {  // uniform: the time-modulated norm, gain 1 + fscale and shift fshift
      const float4 f = *reinterpret_cast<const float4 *>(fscale + c);
      gv[j] = make_float4(1.f + f.x, 1.f + f.y, 1.f + f.z, 1.f + f.w);
      sv[j] = *reinterpret_cast<const float4 *>(fshift + c);
    } else {
      gv[j] = *reinterpret_cast<const float4 *>(gain + c);
      sv[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (4 * tid + 1024 * j >= H) hv[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    ss += hv[j].x * hv[j].x + hv[j].y * hv[j].y + hv[j].z * hv[j].z + hv[j].w * hv[j].w;
  }
  ss = wave_sum(ss);
  if (lane == 0) red1[wave] = ss;
  __syncthreads();
  const float inv = rsqrtf((red1[0] + red1[1] + red1[2] + red1[3]) / H + eps);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (4 * tid + 1024 * j >= H) continue;  // stays zero: a clamped column must add nothing
    hv[j].x = hv[j].x * inv * gv[j].x + sv[j].x; hv[j].y = hv[j].y * inv * gv[j].y + sv[j].y;
    hv[j].z = hv[j].z * inv * gv[j].z + sv[j].z; hv[j].w = hv[j].w * inv * gv[j].w + sv[j].w;
  }
  for (int a0 = 0; a0 < A; a0 += 16) {
    float part[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) part[k] = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (1024 * j >= H) break;  // uniform
      const int c = min(4 * tid + 1024 * j, H - 4);
      float4 wv[16];
#pragma unroll
      for (int k = 0; k < 16; ++k)  // unconditional loads (clamped row) stay in flight together
        wv[k] = *reinterpret_cast<const float4 *>(w_out + (size_t)min(a0 + k, A - 1) * H + c);
#pragma unroll
      for (int k = 0; k < 16; ++k)
        part[k] += wv[k].x * hv[j].x + wv[k].y * hv[j].y + wv[k].z * hv[j].z + wv[k].w * hv[j].w;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float v = wave_sum(part[k]);
      if (lane == 0) red[wave][k] = v;
    }
    __syncthreads();
    if (tid < 16 && a0 + tid < A) {
      const float v = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid] + b_out[a0 + tid];
      x[(size_t)m * A + a0 + tid] -= v * inv_steps;
    }
    __syncthreads();
  }
}
void launch_velocity_euler(const float *h, const float *gain, const float *w_out, const float *b_out, float *x, int M,
                           int H, int A, float eps, int num_steps, hipStream_t s, const float *fscale,
                           const float *fshift) {
  hipLaunchKernelGGL(velocity_euler_kernel, dim3(M), dim3(256), 0, s, h, gain, w_out, b_out, x, H, A, eps,
                     1.0f / (float)num_steps, fscale, fshift);
}

// ---------------------------------------------------------------- time modulation of the action expert
// Page "DM0.5: High-Performance Embodied VLA ...", section 5.2: time_mlp_in / time_mlp_out turn the
// flow time into a modulation signal and every layer's modulator turns it into the scale, shift
// and gate of its two norms.  t is shared by the whole batch, so a chunk's tables (all Euler
// steps, all layers) are computed once before the first step, each weight read once.

// tau[k][i] = sin / cos(t_k * 10000^(-2j/H)) with t_k = 1 - k / num_steps (as in embed_kernel).
__global__ void tau_table_kernel(float *tau, int num_steps, int H) {
  const int k = blockIdx.y, i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= H) return;
  const int half = H / 2, j = i < half ? i : i - half;
  const float t = 1.0f - (float)k / (float)num_steps;
  const float w = exp2f(-2.0f * (float)j / (float)H * 13.287712379549449f);
  tau[(size_t)k * H + i] = i < half ? sinf(t * w) : cosf(t * w);
}
void launch_tau_table(float *tau, int num_steps, int H, hipStream_t s) {
  hipLaunchKernelGGL(tau_table_kernel, dim3((H + 255) / 256, num_steps), dim3(256), 0, s, tau, num_steps, H);
}

// Y[m][n] = b[n] + sum_k f(X[m][k]) W[n][k], M <= 16, K <= 1024 (a multiple of 8): the M input
// rows (f applied) sit in LDS; each wave takes one output row n at a time, its lanes 8 consecutive
// inputs each (one 16- or 32-byte load), then one reduction across the wave per input row.
constexpr int GEMV_MAX_ROWS = 16, GEMV_MAX_K = 1024;
template <typename WT>
__global__ __launch_bounds__(256) void rows_gemv_kernel(const float *__restrict__ X, int M, int K,
                                                        const WT *__restrict__ W, const float *__restrict__ b,
                                                        float *__restrict__ Y, int N, int silu_in) {
  __shared__ float xs[GEMV_MAX_ROWS * GEMV_MAX_K];
  for (int e = threadIdx.x; e < M * K; e += blockDim.x) {
    const float v = X[e];
    xs[e] = silu_in ? silu(v) : v;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  for (int n = blockIdx.x * nwave + wave; n < N; n += gridDim.x * nwave) {
    float acc[GEMV_MAX_ROWS];
#pragma unroll
    for (int m = 0; m < GEMV_MAX_ROWS; ++m) acc[m] = 0.f;
    const WT *wr = W + (size_t)n * K;
    for (int c = lane; c < K / 8; c += 64) {
      float w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = to_f32(wr[8 * c + e]);
#pragma unroll
      for (int m = 0; m < GEMV_MAX_ROWS; ++m)
        if (m < M) {
          const float *xr = xs + m * K + 8 * c;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[m] += w[e] * xr[e];
        }
    }
#pragma unroll
    for (int m = 0; m < GEMV_MAX_ROWS; ++m)
      if (m < M) {
        const float v = wave_sum(acc[m]);
        if (lane == 0) Y[(size_t)m * N + n] = v + b[n];
      }
  }
}
void launch_rows_gemv(Dt dt, const float *X, int M, int K, const void *W, const float *b, float *Y, int N, bool silu_in,
                      hipStream_t s) {
  const int blocks = std::min(1024, (N + 3) / 4);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(rows_gemv_kernel<bf16>, dim3(blocks), dim3(256), 0, s, X, M, K, (const bf16 *)W, b, Y, N,
                       (int)silu_in);
  else
    hipLaunchKernelGGL(rows_gemv_kernel<float>, dim3(blocks), dim3(256), 0, s, X, M, K, (const float *)W, b, Y, N,
                       (int)silu_in);
}

// hg[m][i] = h[m][i] / rms(h[m]) * (1 + scale[i]) + shift[i]: one workgroup per row, thread t the
// columns 4t + 1024j (H <= 4096, a multiple of 4).
template <typename T>
__global__ __launch_bounds__(256) void mod_norm_kernel(const float *__restrict__ h, T *__restrict__ hg,
                                                       const float *__restrict__ scale, const float *__restrict__ shift,
                                                       int H, float eps) {
  __shared__ float red[4];
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float4 hv[4];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = 4 * tid + 1024 * j;
    hv[j] = c < H ? *reinterpret_cast<const float4 *>(h + (size_t)m * H + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    ss += hv[j].x * hv[j].x + hv[j].y * hv[j].y + hv[j].z * hv[j].z + hv[j].w * hv[j].w;
  }
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  const float inv = rsqrtf((red[0] + red[1] + red[2] + red[3]) / H + eps);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = 4 * tid + 1024 * j;
    if (c >= H) continue;
    const float4 sc = *reinterpret_cast<const float4 *>(scale + c), sh = *reinterpret_cast<const float4 *>(shift + c);
    T *o = hg + (size_t)m * H + c;
    o[0] = from_f32<T>(hv[j].x * inv * (1.f + sc.x) + sh.x);
    o[1] = from_f32<T>(hv[j].y * inv * (1.f + sc.y) + sh.y);
    o[2] = from_f32<T>(hv[j].z * inv * (1.f + sc.z) + sh.z);
    o[3] = from_f32<T>(hv[j].w * inv * (1.f + sc.w) + sh.w);
  }
}
void launch_mod_norm(Dt dt, const float *h, void *hg, const float *scale, const float *shift, int M, int H, float eps,
                     hipStream_t s) {
  if (dt == DT_BF16)
    hipLaunchKernelGGL(mod_norm_kernel<bf16>, dim3(M), dim3(256), 0, s, h, (bf16 *)hg, scale, shift, H, eps);
  else
    hipLaunchKernelGGL(mod_norm_kernel<float>, dim3(M), dim3(256), 0, s, h, (float *)hg, scale, shift, H, eps);
}

// Nearest E4M3 (OCP e4m3fn) code of a float32 value, ties to even, saturating at +-448:
// 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; subnormal step 2^-9.  Normal range:
// round the float32 mantissa to 3 bits on the bit pattern (a carry moves into the exponent);
// below 2^-6: round a * 2^9 to an integer, which is the subnormal code (8 = smallest normal).
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(x);
  uint32_t code;
  if (a >= 0.015625f) {  // 2^-6
    const uint32_t au = u & 0x7FFFFFFFu;
    const uint32_t r = au + 0x7FFFFu + ((au >> 20) & 1u);  // RNE at mantissa bit 20
    const int e = (int)(r >> 23) - 127 + 7;
    code = ((uint32_t)e << 3) | ((r >> 20) & 7u);
    if (!(a < 448.f) || code > 0x7Eu) code = 0x7Eu;     // saturate (also catches e > 15)
  } else {
    code = (uint32_t)rintf(a * 512.0f);                 // 0..8, ties to even
  }
  return sign | code;
}

// One wave per row (four rows per workgroup); the row is VPL 16-byte vectors per lane, all loaded
// before the row maximum is reduced.  Codes are e4m3(x / s) with s = max|x| / 448, both divisions
// correctly rounded float32.
template <int VPL>
__global__ __launch_bounds__(256) void fp8_rows_kernel(const bf16 *__restrict__ src, uint8_t *__restrict__ dst,
                                                       float *__restrict__ scales, int rows) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  if (row >= rows) return;  // uniform per wave; no workgroup barrier below
  constexpr int cols = 512 * VPL;
  const bf16x8 *p = reinterpret_cast<const bf16x8 *>(src + (size_t)row * cols);
  bf16x8 v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) v[i] = p[i * 64 + lane];
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(to_f32(v[i][e])));
  mx = wave_max(mx);
  const float s = mx > 0.f ? mx / 448.0f : 1.0f;
  if (lane == 0) scales[row] = s;
  uint2 *q = reinterpret_cast<uint2 *>(dst + (size_t)row * cols);
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo |= e4m3_encode(to_f32(v[i][e]) / s) << (8 * e);
      hi |= e4m3_encode(to_f32(v[i][e + 4]) / s) << (8 * e);
    }
    q[i * 64 + lane] = make_uint2(lo, hi);
  }
}

// Any column count: one workgroup per row.
__global__ __launch_bounds__(256) void fp8_rows_any_kernel(const bf16 *__restrict__ src, uint8_t *__restrict__ dst,
                                                           float *__restrict__ scales, int cols) {
  __shared__ float red[4];
  const bf16 *row = src + (size_t)blockIdx.x * cols;
  float mx = 0.f;
  for (int c = threadIdx.x; c < cols; c += 256) mx = fmaxf(mx, fabsf(to_f32(row[c])));
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = mx > 0.f ? mx / 448.0f : 1.0f;
  if (threadIdx.x == 0) scales[blockIdx.x] = s;
  for (int c = threadIdx.x; c < cols; c += 256) dst[(size_t)blockIdx.x * cols + c] = (uint8_t)e4m3_encode(to_f32(row[c]) / s);
}

void launch_fp8_quantize_rows(const void *src, uint8_t *dst, float *scales, int rows, int cols, hipStream_t s) {
  const bf16 *x = (const bf16 *)src;
  const dim3 g4((rows + 3) / 4), blk(256);
  switch (cols % 512 == 0 ? cols / 512 : 0) {
    case 1: hipLaunchKernelGGL(fp8_rows_kernel<1>, g4, blk, 0, s, x, dst, scales, rows); break;
    case 2: hipLaunchKernelGGL(fp8_rows_kernel<2>, g4, blk, 0, s, x, dst, scales, rows); break;
    case 4: hipLaunchKernelGGL(fp8_rows_kernel<4>, g4, blk, 0, s, x, dst, scales, rows); break;
    case 6: hipLaunchKernelGGL(fp8_rows_kernel<6>, g4, blk, 0, s, x, dst, scales, rows); break;
    case 8: hipLaunchKernelGGL(fp8_rows_kernel<8>, g4, blk, 0, s, x, dst, scales, rows); break;
    case 12: hipLaunchKernelGGL(fp8_rows_kernel<12>, g4, blk, 0, s, x, dst, scales, rows); break;
    case 16: hipLaunchKernelGGL(fp8_rows_kernel<16>, g4, blk, 0, s, x, dst, scales, rows); break;
    default: hipLaunchKernelGGL(fp8_rows_any_kernel, dim3(rows), blk, 0, s, x, dst, scales, cols); break;
  }
}

}  // namespace dm

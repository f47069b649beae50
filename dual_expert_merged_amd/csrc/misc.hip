// Small kernels of the path: RoPE table, counter clearing, entry into the first sublayer
// (h*gain and sums of squares), action_in_proj + time embedding, final norm + action_out_proj +
// Euler update, FP8 E4M3 weight quantisation.
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

__global__ void zero_u32_kernel(unsigned *p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}
void launch_zero_u32(unsigned *p, size_t n, hipStream_t s) {
  if (n == 0) return;
  size_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
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
  sq += __shfl_xor(sq, 1, WAVE);
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
// Also writes hg / sums of squares for the first layer's attention norm.
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const float *__restrict__ x, const float *__restrict__ w_in,
                                                    const float *__restrict__ b_in, Hidden hid,
                                                    const float *__restrict__ gain, int M, int A, float t) {
  constexpr int R = 8;  // action tokens per workgroup
  extern __shared__ float smem[];
  float *tau = smem;       // [H]
  float *xs = smem + hid.H;  // [R][A]
  const int H = hid.H, half = H / 2;
  const int m0 = blockIdx.x * R;
  for (int i = threadIdx.x; i < half; i += 256) {
    const double w = pow(10000.0, -2.0 * i / H);
    tau[i] = (float)sin((double)t * w);
    tau[i + half] = (float)cos((double)t * w);
  }
  for (int j = threadIdx.x; j < R * A; j += 256) xs[j] = (m0 + j / A) < M ? x[(size_t)m0 * A + j] : 0.f;
  __syncthreads();
  const int per_row = H / 8;
  for (int idx = threadIdx.x; idx < R * per_row; idx += 256) {
    const int r = idx / per_row, c0 = (idx - r * per_row) * 8;
    const int m = m0 + r;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float acc = 0.f;
      const float *wr = w_in + (size_t)(c0 + e) * A;
      for (int a = 0; a < A; ++a) acc += wr[a] * xs[r * A + a];
      v[e] = acc + b_in[c0 + e] + tau[c0 + e];
    }
    if (m < M) write_hidden8<T>(hid, gain, m, c0, v, true);
    else {  // keep the pair exchange of write_hidden8 in step
      float sq = 0.f;
      sq += __shfl_xor(sq, 1, WAVE);
    }
  }
}
void launch_embed(Dt dt, const float *x, const float *w_in, const float *b_in, const Hidden &hid, const float *gain,
                  int M, int A, float t, hipStream_t s) {
  const size_t lds = (size_t)(hid.H + 8 * A) * sizeof(float);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(embed_kernel<bf16>, dim3((M + 7) / 8), dim3(256), lds, s, x, w_in, b_in, hid, gain, M, A, t);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3((M + 7) / 8), dim3(256), lds, s, x, w_in, b_in, hid, gain, M, A, t);
}

__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < nw; ++w) t += red[w];
  return t;
}

// Page "DM0.5: High-Performance Embodied VLA ...", sections 5.2-5.3: action_out_proj gives the
// velocity and one explicit Euler step moves x toward t = 0:
//   v = RMSNorm(h; gain) w_out^T + b_out ;  x <- x - v / N.
// One workgroup per action token; each wave computes A/4 outputs with lanes across H.
__global__ __launch_bounds__(256) void velocity_euler_kernel(const float *__restrict__ h, const float *__restrict__ gain,
                                                             const float *__restrict__ w_out,
                                                             const float *__restrict__ b_out, float *__restrict__ x,
                                                             int H, int A, float eps, float inv_steps) {
  __shared__ float red[4];
  extern __shared__ float nrm[];
  const int m = blockIdx.x;
  const float *row = h + (size_t)m * H;
  float ss = 0.f;
  for (int i = threadIdx.x; i < H; i += 256) ss += row[i] * row[i];
  const float inv = rsqrtf(block_sum(ss, red) / H + eps);
  for (int i = threadIdx.x; i < H; i += 256) nrm[i] = row[i] * inv * gain[i];
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int a = wave; a < A; a += 4) {
    float acc = 0.f;
    for (int i = lane; i < H; i += 64) acc += w_out[(size_t)a * H + i] * nrm[i];
    acc = wave_sum(acc);
    if (lane == 0) x[(size_t)m * A + a] -= (acc + b_out[a]) * inv_steps;
  }
}
void launch_velocity_euler(const float *h, const float *gain, const float *w_out, const float *b_out, float *x, int M,
                           int H, int A, float eps, int num_steps, hipStream_t s) {
  hipLaunchKernelGGL(velocity_euler_kernel, dim3(M), dim3(256), H * sizeof(float), s, h, gain, w_out, b_out, x, H, A,
                     eps, 1.0f / (float)num_steps);
}

// Nearest E4M3 (OCP e4m3fn) code of a float32 value, ties to even, saturating at +-448:
// 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; subnormal step 2^-9.
__device__ __forceinline__ uint8_t e4m3_encode(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (!(a > 0.f)) return (uint8_t)sign;
  if (a >= 448.f) return (uint8_t)(sign | 0x7Eu);
  int e;
  frexpf(a, &e);                    // a = f * 2^e, f in [0.5, 1)
  int E = e - 1;                    // binade exponent
  if (E < -6) E = -6;               // subnormals share the smallest normal's step
  const float step = ldexpf(1.0f, E - 3);
  float r = rintf(a / step) * step; // exact division by a power of two; ties to even
  if (r > 448.f) r = 448.f;
  if (r == 0.f) return (uint8_t)sign;
  int er;
  frexpf(r, &er);
  const int Er = er - 1;
  uint32_t code;
  if (Er < -6) {
    code = (uint32_t)(r * 512.0f);  // subnormal: r = m * 2^-9
  } else {
    const uint32_t mant = (uint32_t)((r / ldexpf(1.0f, Er) - 1.0f) * 8.0f);
    code = ((uint32_t)(Er + 7) << 3) | mant;
  }
  return (uint8_t)(sign | code);
}

__global__ __launch_bounds__(256) void fp8_quant_rows_kernel(const bf16 *__restrict__ src, uint8_t *__restrict__ dst,
                                                             float *__restrict__ scales, int cols) {
  __shared__ float red[4];
  const bf16 *row = src + (size_t)blockIdx.x * cols;
  float mx = 0.f;
  for (int c = threadIdx.x; c < cols; c += 256) mx = fmaxf(mx, fabsf(to_f32(row[c])));
  mx = wave_max(mx);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = mx > 0.f ? mx / 448.0f : 1.0f;
  if (threadIdx.x == 0) scales[blockIdx.x] = s;
  for (int c = threadIdx.x; c < cols; c += 256) dst[(size_t)blockIdx.x * cols + c] = e4m3_encode(to_f32(row[c]) / s);
}
void launch_fp8_quantize_rows(const void *src, uint8_t *dst, float *scales, int rows, int cols, hipStream_t s) {
  hipLaunchKernelGGL(fp8_quant_rows_kernel, dim3(rows), dim3(256), 0, s, (const bf16 *)src, dst, scales, cols);
}

}  // namespace dm

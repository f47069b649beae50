// Small kernels of the path: RoPE table, RMSNorm, action_in_proj + time embedding,
// final norm + action_out_proj + Euler update, FP8 E4M3 weight quantisation.
#include "common.h"
#include "kernels.h"

namespace dm {

// (cos, sin) of pos * base^(-2i/D) for every position and pair index, computed in double
// precision once per call and rounded to float: rotate-half RoPE of the Qwen3 experts
// (page "DM0 paper definition vs. Dexbotic code", section 1 names Qwen3).
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
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks < 1024 ? blocks : 1024), dim3(256), 0, s, table,
                     n_pos, D, (double)base);
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

// out[m] = h[m] / sqrt(mean(h[m]^2) + eps) * gain, one workgroup per row.
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float *__restrict__ h, const float *__restrict__ gain,
                                                      T *__restrict__ out, int H, float eps) {
  __shared__ float red[4];
  const float *row = h + (size_t)blockIdx.x * H;
  float ss = 0.f;
  for (int i = threadIdx.x; i < H; i += 256) ss += row[i] * row[i];
  const float inv = rsqrtf(block_sum(ss, red) / H + eps);
  for (int i = threadIdx.x; i < H; i += 256) out[(size_t)blockIdx.x * H + i] = from_f32<T>(row[i] * inv * gain[i]);
}
void launch_rmsnorm(Dt dt, const float *h, const float *gain, void *out, int M, int H, float eps, hipStream_t s) {
  if (dt == DT_BF16)
    hipLaunchKernelGGL(rmsnorm_kernel<bf16>, dim3(M), dim3(256), 0, s, h, gain, (bf16 *)out, H, eps);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3(M), dim3(256), 0, s, h, gain, (float *)out, H, eps);
}

// Page "DM0.5: High-Performance Embodied VLA ...", section 5.2: action_in_proj lifts each
// action vector to the expert width; the flow time enters as sin/cos(t * 10000^(-2i/H)) added
// to every action token.  h[m][i] = sum_a x[m][a] w_in[i][a] + b_in[i] + tau_i(t).
__global__ __launch_bounds__(256) void embed_kernel(const float *__restrict__ x, const float *__restrict__ w_in,
                                                    const float *__restrict__ b_in, float *__restrict__ h,
                                                    int M, int A, int H, float t) {
  constexpr int R = 8;  // action tokens per workgroup
  extern __shared__ float tau[];  // [H] time embedding, then [R][A] inputs
  float *xs = tau + H;
  const int m0 = blockIdx.x * R;
  const int half = H / 2;
  for (int i = threadIdx.x; i < half; i += 256) {
    const double w = pow(10000.0, -2.0 * i / H);
    tau[i] = (float)sin((double)t * w);
    tau[i + half] = (float)cos((double)t * w);
  }
  for (int j = threadIdx.x; j < R * A; j += 256) {
    const int m = m0 + j / A;
    xs[j] = m < M ? x[(size_t)m0 * A + j] : 0.f;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < R * H; idx += 256) {
    const int r = idx / H, i = idx - r * H;
    if (m0 + r >= M) break;
    float acc = 0.f;
    for (int a = 0; a < A; ++a) acc += w_in[(size_t)i * A + a] * xs[r * A + a];
    h[(size_t)(m0 + r) * H + i] = acc + b_in[i] + tau[i];
  }
}
void launch_embed(const float *x, const float *w_in, const float *b_in, float *h, int M, int A, int H, float t,
                  hipStream_t s) {
  const size_t lds = (size_t)(H + 8 * A) * sizeof(float);
  hipLaunchKernelGGL(embed_kernel, dim3((M + 7) / 8), dim3(256), lds, s, x, w_in, b_in, h, M, A, H, t);
}

// Page "DM0.5: High-Performance Embodied VLA ...", sections 5.2-5.3: action_out_proj gives the
// velocity and one explicit Euler step moves x toward t = 0:
//   v = RMSNorm(h; gain) w_out^T + b_out ;  x <- x - v / N.
// One workgroup per action token; 4 lanes per output, 64 outputs at most.
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
  const int a = threadIdx.x >> 2, part = threadIdx.x & 3;
  float acc = 0.f;
  if (a < A)
    for (int i = part; i < H; i += 4) acc += w_out[(size_t)a * H + i] * nrm[i];
  acc += __shfl_xor(acc, 1, WAVE);
  acc += __shfl_xor(acc, 2, WAVE);
  if (a < A && part == 0) {
    const float v = acc + b_out[a];
    x[(size_t)m * A + a] -= v * inv_steps;
  }
}
void launch_velocity_euler(const float *h, const float *gain, const float *w_out, const float *b_out, float *x, int M,
                           int H, int A, float eps, int num_steps, hipStream_t s) {
  hipLaunchKernelGGL(velocity_euler_kernel, dim3(M), dim3(256), H * sizeof(float), s, h, gain, w_out, b_out, x, H, A,
                     eps, 1.0f / (float)num_steps);
}

__global__ void copy_kernel(const float4 *__restrict__ src, float4 *__restrict__ dst, size_t n4) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}
void launch_copy_f32(const float *src, float *dst, size_t n, hipStream_t s) {
  const size_t n4 = n / 4;
  size_t blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const float4 *)src, (float4 *)dst, n4);
}

// Nearest E4M3 (OCP e4m3fn) code of a float32 value, ties to even, saturating at +-448:
// 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; subnormal step 2^-9.
__device__ __forceinline__ uint8_t e4m3_encode(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  float a = fabsf(x);
  if (!(a > 0.f)) return (uint8_t)sign;
  if (a >= 448.f) return (uint8_t)(sign | 0x7Eu);
  int e;
  frexpf(a, &e);                   // a = f * 2^e, f in [0.5, 1)
  int E = e - 1;                   // binade exponent
  if (E < -6) E = -6;              // subnormals share the smallest normal's step
  const float step = ldexpf(1.0f, E - 3);
  const float qn = rintf(a / step); // integer multiple of the step, ties to even (exact division)
  float r = qn * step;
  if (r > 448.f) r = 448.f;
  // encode r
  if (r == 0.f) return (uint8_t)sign;
  int er;
  frexpf(r, &er);
  int Er = er - 1;
  uint32_t code;
  if (Er < -6) {                   // subnormal: r = m * 2^-9, m in 1..7
    code = (uint32_t)(r * 512.0f);
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

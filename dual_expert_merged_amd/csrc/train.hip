// Kernels of the flow-matching training step on one merged layer (dm_train_merged_layer): a
// strided, batched GEMM on the fp32 matrix cores for every product of the forward and the
// backward, and the row / element kernels around it (RMSNorm and its backward, RoPE and its
// inverse, the masked softmax of the action rows and its backward, SwiGLU and its backward,
// the flow-matching interpolation with action_in_proj, the masked squared-error loss, column
// sums for bias and gain gradients).  Every value is fp32; weights of the bf16 models are
// widened exactly on load.
#include "common.h"
#include "kernels.h"

namespace dm {
namespace {

constexpr int TB = 256;  // threads per block of the row / element kernels

template <typename T> __device__ __forceinline__ float ld(const T *p, long i) { return to_f32(p[i]); }

// ------------------------------------------------------------------------------------- GEMM
// C[m][n] = alpha * sum_k A(m, k) B(n, k) + beta * C[m][n] for a 2-level batch z = (zo, zi):
// A(m, k) = A[zo*a.so + zi*a.si + m*a.sm + k*a.sk], B(n, k) = B[zo*b.so + (zi / bdiv)*b.si +
// n*b.sm + k*b.sk], C[m][n] = C[zo*c.so + zi*c.si + m*ldc + n].  BM x BN tiles (64 or 128
// each), four waves of BM/2 x BN/2 (MFMA 16x16x4 fp32 tiles), k-steps of 16 in two LDS buffers
// (k-major, padded rows): the next k-step's operands are loaded into registers while the
// current one multiplies, then stored into the other buffer, one barrier per k-step.  Each
// thread loads runs of 4 elements along the operand's unit-stride axis (one 16- or 8-byte load
// when the run is in range and aligned, else element by element with zero fill), so any M, N,
// K works.
constexpr int GK = 16;

template <typename T> struct Run4 {
  float v[4];
};
// Loads elements (r0 + e) along `fast` (e = 0..3) of operand X at (row, k) coordinates, with
// zero outside [0, R) x [0, K); `kfast` says the run goes along k (else along the rows).
template <typename T>
__device__ __forceinline__ Run4<T> load_run(const T *__restrict__ x, long sm, long sk, int row, int k, bool kfast,
                                            int R, int K) {
  Run4<T> o;
  const long base = (long)row * sm + (long)k * sk;
  const bool full = kfast ? (row < R && k + 3 < K) : (k < K && row + 3 < R);
  const T *p = x + base;
  constexpr int VB = 4 * sizeof(T);
  if (full && ((uintptr_t)p & (VB - 1)) == 0) {
    if constexpr (sizeof(T) == 4) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(p);
      o.v[0] = v[0], o.v[1] = v[1], o.v[2] = v[2], o.v[3] = v[3];
    } else {
      const bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
      o.v[0] = to_f32(v[0]), o.v[1] = to_f32(v[1]), o.v[2] = to_f32(v[2]), o.v[3] = to_f32(v[3]);
    }
    return o;
  }
  const long step = kfast ? sk : sm;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int rr = kfast ? row : row + e, kk = kfast ? k + e : k;
    o.v[e] = (rr < R && kk < K) ? to_f32(x[base + e * step]) : 0.f;
  }
  return o;
}

template <int BM, int BN, typename TA, typename TB_>
__global__ __launch_bounds__(256) void tgemm_kernel(TGemm g, const TA *__restrict__ A, const TB_ *__restrict__ B) {
  constexpr int NA = BM * GK / 1024, NB = BN * GK / 1024;  // 4-element runs per thread per k-step
  constexpr int TM = BM / 32, TN = BN / 32;                // 16x16 tiles per wave
  __shared__ float As[2][GK][BM + 4], Bs[2][GK][BN + 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, c16 = lane & 15, gq = lane >> 4;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  // blockIdx.z = batch index * splits + split; a split takes its own k range and writes raw sums
  // to its slice [batch index][split] of g.part (tgemm_reduce_kernel finishes)
  const int split = blockIdx.z % g.splits, zb = blockIdx.z / g.splits;
  const int zo = zb / g.zi_n, zi = zb - zo * g.zi_n;
  const TA *a = A + zo * g.a.so + zi * g.a.si;
  const TB_ *b = B + zo * g.b.so + (zi / g.bdiv) * g.b.si;
  float *c = g.splits > 1 ? g.part + ((long)zb * g.splits + split) * g.M * g.N : g.C + zo * g.c_so + zi * g.c_si;
  const long ldc = g.splits > 1 ? g.N : g.ldc;
  const float alpha = g.splits > 1 ? 1.f : g.alpha, beta = g.splits > 1 ? 0.f : g.beta;
  const int kb = split * g.k_per_split, ke = min(g.K, kb + g.k_per_split);  // multiple of GK apart
  const bool a_kf = g.a.sk == 1, b_kf = g.b.sk == 1;
  // run q of this thread covers (row, k..k+3) when k-fast, else (row..row+3, k)
  auto coord = [&](int q, bool kf, int rows, int &r, int &k) {
    const int id = q * 256 + tid;
    if (kf) r = id / (GK / 4), k = (id % (GK / 4)) * 4;
    else k = id / (rows / 4), r = (id % (rows / 4)) * 4;
  };
  Run4<TA> ra[NA];
  Run4<TB_> rb[NB];
  auto load = [&](int k0) {
#pragma unroll
    for (int q = 0; q < NA; ++q) {
      int r, k;
      coord(q, a_kf, BM, r, k);
      ra[q] = load_run(a, g.a.sm, g.a.sk, m0 + r, k0 + k, a_kf, g.M, ke);
    }
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      int r, k;
      coord(q, b_kf, BN, r, k);
      rb[q] = load_run(b, g.b.sm, g.b.sk, n0 + r, k0 + k, b_kf, g.N, ke);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int q = 0; q < NA; ++q) {
      int r, k;
      coord(q, a_kf, BM, r, k);
#pragma unroll
      for (int e = 0; e < 4; ++e) As[buf][a_kf ? k + e : k][a_kf ? r : r + e] = ra[q].v[e];
    }
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      int r, k;
      coord(q, b_kf, BN, r, k);
#pragma unroll
      for (int e = 0; e < 4; ++e) Bs[buf][b_kf ? k + e : k][b_kf ? r : r + e] = rb[q].v[e];
    }
  };
  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nk = ke > kb ? (ke - kb + GK - 1) / GK : 0;
  load(kb);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load(kb + (kt + 1) * GK);  // in flight during this k-step's MFMAs
#pragma unroll
    for (int kc = 0; kc < GK / 4; ++kc) {
      float fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[i] = As[cur][kc * 4 + gq][wm * (BM / 2) + i * 16 + c16];
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j] = Bs[cur][kc * 4 + gq][wn * (BN / 2) + j * 16 + c16];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store(cur ^ 1);  // the other buffer was last read before the previous barrier
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * (BM / 2) + i * 16 + 4 * gq + r, n = n0 + wn * (BN / 2) + j * 16 + c16;
        if (m < g.M && n < g.N) {
          float *p = c + (long)m * ldc + n;
          *p = alpha * acc[i][j][r] + (beta != 0.f ? beta * *p : 0.f);
        }
      }
}

// C[m][n] = alpha * sum over splits (in order) of part[z][s][m][n] + beta * C[m][n], every batch
// entry z = (zo, zi)
__global__ __launch_bounds__(256) void tgemm_reduce_kernel(TGemm g) {
  const long mn = (long)g.M * g.N, idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= mn * g.zo_n * g.zi_n) return;
  const long zb = idx / mn, r = idx - zb * mn;
  const int zo = (int)(zb / g.zi_n), zi = (int)(zb - (long)zo * g.zi_n);
  const int m = (int)(r / g.N), n = (int)(r - (long)m * g.N);
  const float *part = g.part + zb * g.splits * mn + r;
  float acc = 0.f;
#pragma unroll 8
  for (int sp = 0; sp < g.splits; ++sp) acc += part[(long)sp * mn];
  float *p = g.C + zo * g.c_so + zi * g.c_si + (long)m * g.ldc + n;
  *p = g.alpha * acc + (g.beta != 0.f ? g.beta * *p : 0.f);
}

// ------------------------------------------------------------------------- row kernels
__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < TB / 64; ++i) s += red[i];
  return s;
}

// y = x * r * g with r = (mean(x^2) + eps)^-1/2 per row; rows past a sample's prefix (when
// `lens` is set: row = b * rows_per_b + j, valid while j < lens[b]) get y = 0 and r = 0.
template <typename TG>
__global__ __launch_bounds__(TB) void rms_fwd_kernel(const float *__restrict__ x, const TG *__restrict__ g, float eps,
                                                     int H, const int *__restrict__ lens, int rows_per_b,
                                                     float *__restrict__ y, float *__restrict__ rstd) {
  __shared__ float red[TB / 64];
  const long row = blockIdx.x;
  const float *xr = x + row * H;
  bool valid = true;
  if (lens) {
    const int b = (int)(row / rows_per_b), j = (int)(row - (long)b * rows_per_b);
    valid = j < lens[b];
  }
  float ss = 0.f;
  for (int i = threadIdx.x; i < H; i += TB) ss += xr[i] * xr[i];
  const float r = valid ? rsqrtf(block_sum(ss, red) / H + eps) : 0.f;
  for (int i = threadIdx.x; i < H; i += TB) y[row * H + i] = valid ? xr[i] * r * ld(g, i) : 0.f;
  if (threadIdx.x == 0) rstd[row] = r;
}

// dx = r (g . dy) - x r^3 sum(g . dy . x) / H per row; out = dx (+ add when set); rows with
// r = 0 (past a prefix) get dx = 0 (r is uniform over the block, so the early exit is too)
template <typename TG>
__global__ __launch_bounds__(TB) void rms_bwd_kernel(const float *__restrict__ x, const TG *__restrict__ g,
                                                     const float *__restrict__ dy, const float *__restrict__ rstd,
                                                     const float *__restrict__ add, int H, float *__restrict__ out) {
  __shared__ float red[TB / 64];
  const long row = blockIdx.x;
  const float r = rstd[row];
  if (r == 0.f) {  // a row past its sample's prefix: no gradient, and its x is never read
    for (int i = threadIdx.x; i < H; i += TB) out[row * H + i] = add ? add[row * H + i] : 0.f;
    return;
  }
  float s = 0.f;
  for (int i = threadIdx.x; i < H; i += TB) s += ld(g, i) * dy[row * H + i] * x[row * H + i];
  const float c = block_sum(s, red) * r * r * r / H;
  for (int i = threadIdx.x; i < H; i += TB) {
    const long k = row * H + i;
    const float dx = r * ld(g, i) * dy[k] - x[k] * c;
    out[k] = add ? add[k] + dx : dx;
  }
}

// Column sums in two passes: partial[c][n] = sum over rows m in chunk c (CS rows) of dy[m][n]
// (* x[m][n] * r[m] when x is set, skipping rows with r = 0), then out[n] = sum over chunks in
// order; deterministic.  A chunk's loads are all issued before its sum, and short chunks give
// the action rows' sums (50 rows) more than a handful of workgroups.
constexpr int CS = 16;
__global__ __launch_bounds__(TB) void colsum_part_kernel(const float *__restrict__ dy, const float *__restrict__ x,
                                                         const float *__restrict__ rstd, int M, int N,
                                                         float *__restrict__ part) {
  const int n = blockIdx.x * TB + threadIdx.x;
  if (n >= N) return;
  const int m0 = blockIdx.y * CS;
  float t[CS];
#pragma unroll
  for (int j = 0; j < CS; ++j) {
    const int m = m0 + j;
    const long k = (long)m * N + n;
    t[j] = 0.f;
    if (m < M) {
      if (!x) t[j] = dy[k];
      else {
        const float r = rstd[m];
        t[j] = r != 0.f ? dy[k] * x[k] * r : 0.f;
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < CS; ++j) s += t[j];
  part[(long)blockIdx.y * N + n] = s;
}
__global__ __launch_bounds__(TB) void colsum_final_kernel(const float *__restrict__ part, int chunks, int N,
                                                          float *__restrict__ out) {
  const int n = blockIdx.x * TB + threadIdx.x;
  if (n >= N) return;
  float s = 0.f;
#pragma unroll 8
  for (int c = 0; c < chunks; ++c) s += part[(long)c * N + n];
  out[n] = s;
}

// Rotate-half RoPE in place on `heads` head vectors of D starting at column col0 of rows of
// width ld; row = b * rows_per_b + j sits at position j (+ lens[b] when after_prefix); sign -1
// applies the inverse rotation.  Angles in double: pos * base^(-2i/D).
__global__ __launch_bounds__(TB) void rope_kernel(float *__restrict__ p, long rows, int rows_per_b, int ld, int col0,
                                                  int heads, int D, double base, const int *__restrict__ lens,
                                                  bool after_prefix, float sign) {
  const int half = D / 2;
  const long idx = (long)blockIdx.x * TB + threadIdx.x;
  if (idx >= rows * heads * half) return;
  const int i = (int)(idx % half);
  const long rh = idx / half;
  const int h = (int)(rh % heads);
  const long row = rh / heads;
  const int b = (int)(row / rows_per_b), j = (int)(row - (long)b * rows_per_b);
  const double pos = (double)j + (after_prefix ? (double)lens[b] : 0.0);
  const double ang = pos * pow(base, -2.0 * i / D);
  const float cs = (float)cos(ang), sn = sign * (float)sin(ang);
  float *v = p + row * ld + col0 + (long)h * D;
  const float u1 = v[i], u2 = v[i + half];
  v[i] = u1 * cs - u2 * sn;
  v[i + half] = u2 * cs + u1 * sn;
}

// Joined keys / values [B][Hkv][T][D], T = P_cap + S: rows j < lens[b] from the prefix
// projection kvp [B*P_cap][2 Hkv D] (keys then values), rows P_cap + s from the action rows'
// qkv [B*S][QKV] (keys at column Hq D, values after); the rows in between are zero.
__global__ __launch_bounds__(TB) void gather_kv_kernel(const float *__restrict__ kvp, const float *__restrict__ qkv,
                                                       const int *__restrict__ lens, int B, int P_cap, int S, int Hq,
                                                       int Hkv, int D, float *__restrict__ K, float *__restrict__ V) {
  const int T = P_cap + S;
  const long idx = (long)blockIdx.x * TB + threadIdx.x;
  if (idx >= (long)B * Hkv * T * D) return;
  const int d = (int)(idx % D);
  const long r = idx / D;
  const int j = (int)(r % T);
  const int g = (int)((r / T) % Hkv), b = (int)(r / ((long)T * Hkv));
  float kv = 0.f, vv = 0.f;
  if (j < P_cap) {
    if (j < lens[b]) {
      const float *src = kvp + ((long)b * P_cap + j) * 2 * Hkv * D;
      kv = src[g * D + d];
      vv = src[(Hkv + g) * D + d];
    }
  } else {
    const float *src = qkv + ((long)b * S + (j - P_cap)) * (Hq + 2 * Hkv) * D;
    kv = src[(Hq + g) * D + d];
    vv = src[(Hq + Hkv + g) * D + d];
  }
  K[idx] = kv;
  V[idx] = vv;
}

// The reverse of gather_kv_kernel for gradients: action rows of dK / dV into the key / value
// columns of dqkv, prefix rows j < lens[b] into dkvp (when set; other prefix rows get 0).
__global__ __launch_bounds__(TB) void scatter_kv_kernel(const float *__restrict__ dK, const float *__restrict__ dV,
                                                        const int *__restrict__ lens, int B, int P_cap, int S, int Hq,
                                                        int Hkv, int D, float *__restrict__ dqkv,
                                                        float *__restrict__ dkvp) {
  const int T = P_cap + S;
  const long idx = (long)blockIdx.x * TB + threadIdx.x;
  if (idx >= (long)B * Hkv * T * D) return;
  const int d = (int)(idx % D);
  const long r = idx / D;
  const int j = (int)(r % T);
  const int g = (int)((r / T) % Hkv), b = (int)(r / ((long)T * Hkv));
  if (j < P_cap) {
    if (!dkvp) return;
    float *dst = dkvp + ((long)b * P_cap + j) * 2 * Hkv * D;
    const bool ok = j < lens[b];
    dst[g * D + d] = ok ? dK[idx] : 0.f;
    dst[(Hkv + g) * D + d] = ok ? dV[idx] : 0.f;
  } else {
    float *dst = dqkv + ((long)b * S + (j - P_cap)) * (Hq + 2 * Hkv) * D;
    dst[(Hq + g) * D + d] = dK[idx];
    dst[(Hq + Hkv + g) * D + d] = dV[idx];
  }
}

// Softmax of one score row (sample b, head h, action row s) over the visible keys: prefix rows
// j < lens[b] and the S action rows j >= P_cap; other entries become 0.  In place.
__global__ __launch_bounds__(TB) void softmax_rows_kernel(float *__restrict__ sc, const int *__restrict__ lens,
                                                          int Hq, int S, int P_cap) {
  __shared__ float red[TB / 64];
  const int T = P_cap + S;
  const long row = blockIdx.x;
  const int b = (int)(row / ((long)Hq * S));
  const int P = lens[b];
  float *p = sc + row * T;
  float mx = -INFINITY;
  for (int j = threadIdx.x; j < T; j += TB)
    if (j < P || j >= P_cap) mx = fmaxf(mx, p[j]);
  mx = wave_max(mx);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) red[w] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float s = 0.f;
  for (int j = threadIdx.x; j < T; j += TB) {
    const float e = (j < P || j >= P_cap) ? expf(p[j] - mx) : 0.f;
    p[j] = e;
    s += e;
  }
  const float inv = 1.0f / block_sum(s, red);
  for (int j = threadIdx.x; j < T; j += TB) p[j] *= inv;
}

// dS = P . (dP - sum_j P dP) * scale per row, in place over dP
__global__ __launch_bounds__(TB) void softmax_bwd_kernel(const float *__restrict__ pr, float *__restrict__ dp, int T,
                                                         float scale) {
  __shared__ float red[TB / 64];
  const long row = blockIdx.x;
  const float *p = pr + row * T;
  float *d = dp + row * T;
  float s = 0.f;
  for (int j = threadIdx.x; j < T; j += TB) s += p[j] * d[j];
  const float dot = block_sum(s, red);
  for (int j = threadIdx.x; j < T; j += TB) d[j] = p[j] * (d[j] - dot) * scale;
}

// ------------------------------------------------------------------------- element kernels
// Per action row (b, s): x = t eps + (1 - t) a, u = eps - a, and
// h0 = x W_in^T + b_in + tau(t) with tau_i = sin(t w_i), tau_{i+H/2} = cos(t w_i), w_i = base^(-2i/H).
__global__ __launch_bounds__(TB) void fm_embed_kernel(const float *__restrict__ a, const float *__restrict__ eps,
                                                      const float *__restrict__ t, const float *__restrict__ w_in,
                                                      const float *__restrict__ b_in, int S, int A, int H,
                                                      float time_base, float *__restrict__ x, float *__restrict__ u,
                                                      float *__restrict__ h0) {
  __shared__ float xs[64];
  const long row = blockIdx.x;
  const float tb = t[row / S];
  for (int k = threadIdx.x; k < A; k += TB) {
    const float av = a[row * A + k], ev = eps[row * A + k];
    const float xv = tb * ev + (1.0f - tb) * av;
    xs[k] = xv;
    x[row * A + k] = xv;
    u[row * A + k] = ev - av;
  }
  __syncthreads();
  const int half = H / 2;
  for (int n = threadIdx.x; n < H; n += TB) {
    float acc = 0.f;
    for (int k = 0; k < A; ++k) acc += xs[k] * w_in[(long)n * A + k];
    const int i = n < half ? n : n - half;
    const float arg = tb * powf(time_base, -2.0f * i / H);
    h0[row * H + n] = acc + b_in[n] + (n < half ? sinf(arg) : cosf(arg));
  }
}

// dst[m][n] = src[m][n] (+ bias[n] when set); src may be NULL (then bias only)
__global__ __launch_bounds__(TB) void copy_bias_kernel(const float *__restrict__ src, const float *__restrict__ bias,
                                                       long M, int N, float *__restrict__ dst) {
  const long idx = (long)blockIdx.x * TB + threadIdx.x;
  if (idx >= M * N) return;
  const int n = (int)(idx % N);
  dst[idx] = (src ? src[idx] : 0.f) + (bias ? bias[n] : 0.f);
}

__global__ __launch_bounds__(TB) void fill_kernel(float *__restrict__ p, long n, float v) {
  const long idx = (long)blockIdx.x * TB + threadIdx.x;
  if (idx < n) p[idx] = v;
}

__global__ __launch_bounds__(TB) void swiglu_fwd_kernel(const float *__restrict__ gt, const float *__restrict__ up,
                                                        long n, float *__restrict__ act) {
  const long i = (long)blockIdx.x * TB + threadIdx.x;
  if (i < n) act[i] = gt[i] / (1.0f + expf(-gt[i])) * up[i];
}

// dgt = dact . up . silu'(gt), dup = dact . silu(gt); silu'(z) = s (1 + z (1 - s)), s = sigmoid(z)
__global__ __launch_bounds__(TB) void swiglu_bwd_kernel(const float *__restrict__ gt, const float *__restrict__ up,
                                                        const float *__restrict__ dact, long n, float *__restrict__ dgt,
                                                        float *__restrict__ dup) {
  const long i = (long)blockIdx.x * TB + threadIdx.x;
  if (i >= n) return;
  const float z = gt[i], s = 1.0f / (1.0f + expf(-z));
  dgt[i] = dact[i] * up[i] * s * (1.0f + z * (1.0f - s));
  dup[i] = dact[i] * z * s;
}

// One workgroup: n_valid = sum(mask), loss = sum(mask (v - u)^2) / n_valid (0 without a valid
// entry), dv = 2 mask (v - u) / n_valid.  Sums run in a fixed order (bitwise reproducible).
__global__ __launch_bounds__(1024) void fm_loss_kernel(const float *__restrict__ v, const float *__restrict__ u,
                                                       const float *__restrict__ mask, long n, float *__restrict__ loss,
                                                       float *__restrict__ dv) {
  __shared__ float red[2][16];
  float sm = 0.f, se = 0.f;
  for (long i = threadIdx.x; i < n; i += 1024) {
    const float e = v[i] - u[i];
    sm += mask[i];
    se += mask[i] * e * e;
  }
  sm = wave_sum(sm);
  se = wave_sum(se);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) red[0][w] = sm, red[1][w] = se;
  __syncthreads();
  float tm = 0.f, te = 0.f;
  for (int i = 0; i < 16; ++i) tm += red[0][i], te += red[1][i];
  const float c = tm > 0.f ? 2.0f / tm : 0.f;
  for (long i = threadIdx.x; i < n; i += 1024) dv[i] = c * mask[i] * (v[i] - u[i]);
  if (threadIdx.x == 0) *loss = tm > 0.f ? te / tm : 0.f;
}

unsigned blocks(long n) { return (unsigned)((n + TB - 1) / TB); }

}  // namespace

// ------------------------------------------------------------------------------- launchers

// Tile shape: the largest of 128 x 128, 128 x 64, 64 x 128 whose grid still gives about one
// workgroup per CU (>= 200), else 64 x 64.  A product with fewer than two workgroups per CU
// splits K (at least 64 per split) until about four per CU (1024 workgroups), the most the
// registers of the 128 x 64 tile allow: one workgroup per CU is four waves, one per SIMD, and
// each k-step's loads then wait out a whole memory round trip.  g.part holds the partial sums
// (batch entries x splits x M x N floats, at most g.part_floats); the reduce runs in split
// order.  Measured on the one-layer DM0-base step (same box, interleaved runs): splitting only
// below 128 workgroups up to 256 1.45 ms, up to 1024 1.22 ms; k-steps of 32 instead of 16 no
// faster (1.47 ms).
template <typename TA, typename TB_>
static void tgemm_t(TGemm g, const void *A, const void *B, hipStream_t s) {
  const long z = (long)g.zo_n * g.zi_n;
  auto tiles = [&](int bm, int bn) { return ((g.M + bm - 1) / bm) * (long)((g.N + bn - 1) / bn); };
  int bm = 64, bn = 64;
  if (g.M > 64 && g.N > 64 && z * tiles(128, 128) >= 200) bm = 128, bn = 128;
  else if (g.M > 64 && z * tiles(128, 64) >= 200) bm = 128;
  else if (g.N > 64 && z * tiles(64, 128) >= 200) bn = 128;
  const long t = z * tiles(bm, bn);
  int splits = 1;
  if (g.part && t < 512)
    while (t * splits * 2 <= 1024 && g.K / (splits * 2) >= 64 &&
           (size_t)(z * splits * 2) * g.M * g.N <= g.part_floats)
      splits *= 2;
  g.splits = splits;
  g.k_per_split = (((g.K + splits - 1) / splits) + GK - 1) / GK * GK;
  dim3 grid((g.N + bn - 1) / bn, (g.M + bm - 1) / bm, (unsigned)(z * splits));
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, g, (const TA *)A, (const TB_ *)B); };
  if (bm == 128 && bn == 128) go(tgemm_kernel<128, 128, TA, TB_>);
  else if (bm == 128) go(tgemm_kernel<128, 64, TA, TB_>);
  else if (bn == 128) go(tgemm_kernel<64, 128, TA, TB_>);
  else go(tgemm_kernel<64, 64, TA, TB_>);
  if (splits > 1)
    hipLaunchKernelGGL(tgemm_reduce_kernel, dim3(blocks(z * g.M * g.N)), dim3(256), 0, s, g);
}
void launch_tgemm(const TGemm &g, Dt ta, const void *A, Dt tb, const void *B, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.zo_n <= 0 || g.zi_n <= 0) return;
  if (ta == DT_F32 && tb == DT_F32) tgemm_t<float, float>(g, A, B, s);
  else if (ta == DT_F32) tgemm_t<float, bf16>(g, A, B, s);
  else if (tb == DT_F32) tgemm_t<bf16, float>(g, A, B, s);
  else tgemm_t<bf16, bf16>(g, A, B, s);
}
void launch_rms_fwd(const float *x, Dt gt, const void *g, float eps, long rows, int H, const int *lens, int rows_per_b,
                    float *y, float *rstd, hipStream_t s) {
  if (gt == DT_BF16)
    hipLaunchKernelGGL(rms_fwd_kernel<bf16>, dim3(rows), dim3(TB), 0, s, x, (const bf16 *)g, eps, H, lens, rows_per_b, y,
                       rstd);
  else
    hipLaunchKernelGGL(rms_fwd_kernel<float>, dim3(rows), dim3(TB), 0, s, x, (const float *)g, eps, H, lens, rows_per_b,
                       y, rstd);
}
void launch_rms_bwd(const float *x, Dt gt, const void *g, const float *dy, const float *rstd, const float *add, long rows,
                    int H, float *out, hipStream_t s) {
  if (gt == DT_BF16)
    hipLaunchKernelGGL(rms_bwd_kernel<bf16>, dim3(rows), dim3(TB), 0, s, x, (const bf16 *)g, dy, rstd, add, H, out);
  else
    hipLaunchKernelGGL(rms_bwd_kernel<float>, dim3(rows), dim3(TB), 0, s, x, (const float *)g, dy, rstd, add, H, out);
}
void launch_colsum(const float *dy, const float *x, const float *rstd, int M, int N, float *out, float *part,
                   hipStream_t s) {
  const int chunks = (M + CS - 1) / CS;
  hipLaunchKernelGGL(colsum_part_kernel, dim3(blocks(N), chunks), dim3(TB), 0, s, dy, x, rstd, M, N, part);
  hipLaunchKernelGGL(colsum_final_kernel, dim3(blocks(N)), dim3(TB), 0, s, part, chunks, N, out);
}
size_t colsum_part_floats(int M, int N) { return (size_t)((M + CS - 1) / CS) * N; }
void launch_rope_rows(float *p, long rows, int rows_per_b, int ld, int col0, int heads, int D, double base,
                      const int *lens, bool after_prefix, float sign, hipStream_t s) {
  hipLaunchKernelGGL(rope_kernel, dim3(blocks(rows * heads * (D / 2))), dim3(TB), 0, s, p, rows, rows_per_b, ld, col0,
                     heads, D, base, lens, after_prefix, sign);
}
void launch_gather_kv(const float *kvp, const float *qkv, const int *lens, int B, int P_cap, int S, int Hq, int Hkv,
                      int D, float *K, float *V, hipStream_t s) {
  hipLaunchKernelGGL(gather_kv_kernel, dim3(blocks((long)B * Hkv * (P_cap + S) * D)), dim3(TB), 0, s, kvp, qkv, lens, B,
                     P_cap, S, Hq, Hkv, D, K, V);
}
void launch_scatter_kv(const float *dK, const float *dV, const int *lens, int B, int P_cap, int S, int Hq, int Hkv,
                       int D, float *dqkv, float *dkvp, hipStream_t s) {
  hipLaunchKernelGGL(scatter_kv_kernel, dim3(blocks((long)B * Hkv * (P_cap + S) * D)), dim3(TB), 0, s, dK, dV, lens, B,
                     P_cap, S, Hq, Hkv, D, dqkv, dkvp);
}
void launch_softmax_rows(float *sc, const int *lens, int B, int Hq, int S, int P_cap, hipStream_t s) {
  hipLaunchKernelGGL(softmax_rows_kernel, dim3((unsigned)((long)B * Hq * S)), dim3(TB), 0, s, sc, lens, Hq, S, P_cap);
}
void launch_softmax_bwd(const float *p, float *dp, long rows, int T, float scale, hipStream_t s) {
  hipLaunchKernelGGL(softmax_bwd_kernel, dim3((unsigned)rows), dim3(TB), 0, s, p, dp, T, scale);
}
void launch_fm_embed(const float *a, const float *eps, const float *t, const float *w_in, const float *b_in, int B, int S,
                     int A, int H, float time_base, float *x, float *u, float *h0, hipStream_t s) {
  hipLaunchKernelGGL(fm_embed_kernel, dim3((unsigned)((long)B * S)), dim3(TB), 0, s, a, eps, t, w_in, b_in, S, A, H,
                     time_base, x, u, h0);
}
void launch_copy_bias(const float *src, const float *bias, long M, int N, float *dst, hipStream_t s) {
  hipLaunchKernelGGL(copy_bias_kernel, dim3(blocks(M * N)), dim3(TB), 0, s, src, bias, M, N, dst);
}
void launch_fill(float *p, long n, float v, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(fill_kernel, dim3(blocks(n)), dim3(TB), 0, s, p, n, v);
}
void launch_swiglu_fwd(const float *gt, const float *up, long n, float *act, hipStream_t s) {
  hipLaunchKernelGGL(swiglu_fwd_kernel, dim3(blocks(n)), dim3(TB), 0, s, gt, up, n, act);
}
void launch_swiglu_bwd(const float *gt, const float *up, const float *dact, long n, float *dgt, float *dup, hipStream_t s) {
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(blocks(n)), dim3(TB), 0, s, gt, up, dact, n, dgt, dup);
}
void launch_fm_loss(const float *v, const float *u, const float *mask, long n, float *loss, float *dv, hipStream_t s) {
  hipLaunchKernelGGL(fm_loss_kernel, dim3(1), dim3(1024), 0, s, v, u, mask, n, loss, dv);
}

}  // namespace dm

// Dense projections of the merged layer on gfx950 MFMA: C = A W^T, A token-major activations
// [M][K] in the weight dtype, W in the [out][in] layout, fp32 accumulation, fused epilogues:
//   qkv    : RMSNorm row scale, RoPE on query/key columns, scatter to queries and head-major K/V
//   resid  : h += C (fp32 residual stream), then the next sublayer's h*gain and sums of squares
//   swiglu : RMSNorm row scale, act = silu(gate) * up
// Page "DM0 paper definition vs. Dexbotic code", section 1: each expert applies its own Q/K/V,
// O-projection + residual and MLP; "DM0.5: High-Performance Embodied VLA ...", section 6.3
// names gate/up/down as the MLP GEMMs.
//
// RMSNorm is folded in: the producer of h writes hg = h*gain (rounded to the weight dtype) and
// per-16-column sums of squares; the consumer runs the GEMM on hg and multiplies each output row
// by 1/sqrt(mean(h^2) + eps), which is RMSNorm(h) W^T up to the rounding of hg.
//
// Two kernels share the epilogues:
//  * skinny (M <= 64, the batch-1 action chunk): one workgroup owns NT output columns for all
//    rows and one K slice; its 4 waves each take a quarter of the slice and load MFMA fragments
//    straight from global memory (16 bytes per lane, four k-chunks in flight), then reduce
//    through LDS.  Narrow-N GEMMs also split K across workgroups: each writes an fp32 partial
//    tile, and the last to arrive (arrival counter) sums the partials in split order, so results
//    do not depend on scheduling, and runs the epilogue.
//  * tiled (larger M): a 64x64 output tile per workgroup, A and W staged through LDS.
// Column permutations put the two halves of every RoPE pair, and the gate/up pair of every
// SwiGLU column, in lanes l and l^8 of one MFMA tile, so one cross-lane exchange joins them.
#include "common.h"
#include "kernels.h"

namespace dm {

__device__ __forceinline__ bool row_valid(const RowMap &rm, int row, int M, int *b_out, int *s_out) {
  if (row >= M) return false;
  const int b = row / rm.rows_per_b, s = row - b * rm.rows_per_b;
  *b_out = b;
  *s_out = s;
  return rm.is_prefix ? (s < max(0, min(rm.lens[b], rm.cap))) : true;
}

// 1/rms of rows m0..m0+63 into inv[64], from per-16-column sums of squares; 4 threads per row,
// fixed summation order.
__device__ __forceinline__ void rms_prepare(const Hidden &in, int M, float eps, int m0, float *inv) {
  const int t = threadIdx.x, row = t >> 2, part = t & 3;
  const int nt = in.H >> 4;
  float s = 0.f;
  const int m = m0 + row;
  if (m < M)
    for (int i = part; i < nt; i += 4) s += in.ssq[(size_t)m * nt + i];
  s += __shfl_xor(s, 1, WAVE);
  s += __shfl_xor(s, 2, WAVE);
  if (part == 0) inv[row] = rsqrtf(s / (float)in.H + eps);
}

template <typename T> struct EpiQkv {
  QkvArgs a;
  __device__ __forceinline__ int col(int c) const {
    const int qd = a.Hq * a.D, kd = a.Hkv * a.D;
    const int base = c < qd ? 0 : (c < qd + kd ? qd : qd + kd);
    const int local = c - base;
    const int half = a.D >> 1;
    const int p = (local >> 4) * 8 + (local & 7);
    const int upper = (local >> 3) & 1;
    return base + (p / half) * a.D + (p % half) + upper * half;
  }
  __device__ __forceinline__ const T *wrow(int c) const { return (const T *)a.w + (size_t)col(c) * a.in.H; }
  __device__ __forceinline__ void prepare(int m0, float *inv) const { rms_prepare(a.in, a.M, a.eps, m0, inv); }

  __device__ __forceinline__ void tile(int row0, int c, f32x4 acc, const float *inv, int m0) const {
    const int gc = col(c);
    const int D = a.D, qd = a.Hq * D, kd = a.Hkv * D;
    const int sec = gc < qd ? 0 : (gc < qd + kd ? 1 : 2);
    const int local = gc - (sec == 0 ? 0 : (sec == 1 ? qd : qd + kd));
    const int head = local / D, d = local - head * D;
    const int half = D >> 1;
    const int upper = d >= half;
    const int i = d - upper * half;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float u = acc[r] * inv[row0 + r - m0];
      const float pu = __shfl_xor(u, 8, WAVE);
      int b, s;
      if (!row_valid(a.rows, row0 + r, a.M, &b, &s)) continue;
      if (sec < 2) {
        const int pos = a.rows.is_prefix ? s : max(0, min(a.rows.lens[b], a.rows.cap)) + s;
        const float2 cs = a.rope[(size_t)pos * half + i];
        u = upper ? (u * cs.x + pu * cs.y) : (u * cs.x - pu * cs.y);
      }
      const T val = from_f32<T>(u);
      if (sec == 0) {
        ((T *)a.q)[(size_t)(row0 + r) * qd + gc] = val;
      } else {
        T *dst = (T *)(sec == 1 ? a.k : a.v);
        dst[((size_t)(b * a.Hkv + head) * a.kv_rows + s) * D + d] = val;
      }
    }
  }
};

template <typename T> struct EpiResid {
  ResidArgs a;
  __device__ __forceinline__ const T *wrow(int c) const { return (const T *)a.w + (size_t)c * a.K; }
  __device__ __forceinline__ void prepare(int, float *) const {}
  __device__ __forceinline__ void tile(int row0, int c, f32x4 acc, const float *, int) const {
    const int H = a.out.H;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + r;
      int b, s;
      const bool ok = row_valid(a.rows, row, a.M, &b, &s);
      float hn = 0.f;
      if (ok) {
        hn = a.out.h[(size_t)row * H + c] + acc[r];
        a.out.h[(size_t)row * H + c] = hn;
        if (a.next_gain) ((T *)a.out.hg)[(size_t)row * H + c] = from_f32<T>(hn * a.next_gain[c]);
      }
      if (a.next_gain) {
        float sq = hn * hn;
        sq += __shfl_xor(sq, 1, WAVE);
        sq += __shfl_xor(sq, 2, WAVE);
        sq += __shfl_xor(sq, 4, WAVE);
        sq += __shfl_xor(sq, 8, WAVE);
        if (ok && (c & 15) == 0) a.out.ssq[(size_t)row * (H >> 4) + (c >> 4)] = sq;
      }
    }
  }
};

template <typename T> struct EpiSwiglu {
  SwigluArgs a;
  __device__ __forceinline__ const T *wrow(int c) const {
    const int f = (c >> 4) * 8 + (c & 7);
    return (const T *)((c >> 3) & 1 ? a.wu : a.wg) + (size_t)f * a.in.H;
  }
  __device__ __forceinline__ void prepare(int m0, float *inv) const { rms_prepare(a.in, a.M, a.eps, m0, inv); }
  __device__ __forceinline__ void tile(int row0, int c, f32x4 acc, const float *inv, int m0) const {
    const int f = (c >> 4) * 8 + (c & 7);
    const int up = (c >> 3) & 1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float g = acc[r] * inv[row0 + r - m0];
      const float u = __shfl_xor(g, 8, WAVE);
      int b, s;
      if (up || !row_valid(a.rows, row0 + r, a.M, &b, &s)) continue;
      ((T *)a.act)[(size_t)(row0 + r) * a.F + f] = from_f32<T>(silu(g) * u);
    }
  }
};

// ------------------------------------------------------------------------ skinny kernel (M <= 64)
template <typename T, int NT, class Epi>
__global__ __launch_bounds__(256) void skinny_kernel(const T *__restrict__ A, int M, int K, Epi epi, SplitK sk) {
  typedef Mfma<T> MF;
  typedef typename MF::frag frag;
  constexpr int EPL = MF::EPL, KC = 4 * EPL, CT = NT / 16, U = 4;
  __shared__ __attribute__((aligned(16))) f32x4 red[4 * 4 * CT * 64];
  __shared__ float rinv[64];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int tile = blockIdx.x, split = blockIdx.y, mt = blockIdx.z, m0 = mt * 64;
  const int n0 = tile * NT;
  const int Ks = K / sk.k_split, Kw = Ks >> 2;
  const int k0 = split * Ks + wave * Kw;
  const int nk = Kw / KC;
  const int nrt = min(4, (M - m0 + 15) >> 4);  // row tiles holding valid rows (uniform)

  epi.prepare(m0, rinv);

  const T *wp[CT];
#pragma unroll
  for (int j = 0; j < CT; ++j) wp[j] = epi.wrow(n0 + j * 16 + c16) + k0 + g * EPL;
  const T *ap[4];
  bool aok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + i * 16 + c16;
    aok[i] = row < M;
    ap[i] = A + (size_t)(aok[i] ? row : 0) * K + k0 + g * EPL;
  }

  f32x4 acc[4][CT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < CT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kc = 0; kc < nk; kc += U) {
    frag wf[U][CT], af[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (kc + u < nk) {
#pragma unroll
        for (int j = 0; j < CT; ++j) wf[u][j] = load_frag<T>(wp[j] + (kc + u) * KC);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          af[u][i] = (i < nrt && aok[i]) ? load_frag<T>(ap[i] + (kc + u) * KC) : zero_frag<T>();
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (kc + u < nk) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i < nrt)
#pragma unroll
            for (int j = 0; j < CT; ++j) acc[i][j] = MF::mma(af[u][i], wf[u][j], acc[i][j]);
      }
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < CT; ++j) red[((wave * 4 + i) * CT + j) * 64 + lane] = acc[i][j];
  __syncthreads();
  f32x4 sum[CT];
#pragma unroll
  for (int j = 0; j < CT; ++j) {
    f32x4 t = red[((0 * 4 + wave) * CT + j) * 64 + lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) t += red[((w * 4 + wave) * CT + j) * 64 + lane];
    sum[j] = t;
  }

  if (sk.k_split > 1) {
    const size_t tile_id = (size_t)mt * gridDim.x + tile;
    f32x4 *part = reinterpret_cast<f32x4 *>(sk.part) + tile_id * sk.k_split * (4 * CT * 64);
#pragma unroll
    for (int j = 0; j < CT; ++j) part[(size_t)split * (4 * CT * 64) + (wave * CT + j) * 64 + lane] = sum[j];
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(&sk.counters[tile_id], 1u) == (unsigned)(sk.k_split - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();
#pragma unroll
    for (int j = 0; j < CT; ++j) {
      f32x4 t = part[(wave * CT + j) * 64 + lane];
      for (int sp = 1; sp < sk.k_split; ++sp) t += part[(size_t)sp * (4 * CT * 64) + (wave * CT + j) * 64 + lane];
      sum[j] = t;
    }
    if (tid == 0) sk.counters[tile_id] = 0u;
  }
  if (wave < nrt) {
#pragma unroll
    for (int j = 0; j < CT; ++j) epi.tile(m0 + wave * 16 + 4 * g, n0 + j * 16 + c16, sum[j], rinv, m0);
  }
}

// ------------------------------------------------------------------------ tiled kernel (any M)
template <typename T, class Epi>
__global__ __launch_bounds__(256) void tiled_kernel(const T *__restrict__ A, int M, int K, Epi epi) {
  typedef Mfma<T> MF;
  typedef typename MF::frag frag;
  constexpr int BM = 64, BN = 64;
  constexpr int EPL = MF::EPL;
  constexpr int KC = 4 * EPL;
  constexpr int BK = 2 * KC;
  constexpr int VPR = BK / EPL;
  constexpr int LDR = BK + EPL;
  constexpr int TM = BM / 32, TN = BN / 32;
  constexpr int AV = BM * VPR / 256, WV = BN * VPR / 256;
  __shared__ __attribute__((aligned(16))) T As[BM * LDR];
  __shared__ __attribute__((aligned(16))) T Ws[BN * LDR];
  __shared__ float rinv[64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  epi.prepare(m0, rinv);

  const T *asrc[AV];
  bool aok[AV];
  int adst[AV];
#pragma unroll
  for (int v = 0; v < AV; ++v) {
    const int idx = tid + v * 256, r = idx / VPR, cv = idx % VPR;
    aok[v] = (m0 + r) < M;
    asrc[v] = A + (size_t)(aok[v] ? m0 + r : 0) * K + cv * EPL;
    adst[v] = r * LDR + cv * EPL;
  }
  const T *wsrc[WV];
  int wdst[WV];
#pragma unroll
  for (int v = 0; v < WV; ++v) {
    const int idx = tid + v * 256, r = idx / VPR, cv = idx % VPR;
    wsrc[v] = epi.wrow(n0 + r) + cv * EPL;
    wdst[v] = r * LDR + cv * EPL;
  }

  frag ra[AV], rw[WV];
  auto gload = [&](int k0) {
#pragma unroll
    for (int v = 0; v < AV; ++v) ra[v] = aok[v] ? load_frag<T>(asrc[v] + k0) : zero_frag<T>();
#pragma unroll
    for (int v = 0; v < WV; ++v) rw[v] = load_frag<T>(wsrc[v] + k0);
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  for (int k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();
#pragma unroll
    for (int v = 0; v < AV; ++v) *reinterpret_cast<frag *>(&As[adst[v]]) = ra[v];
#pragma unroll
    for (int v = 0; v < WV; ++v) *reinterpret_cast<frag *>(&Ws[wdst[v]]) = rw[v];
    __syncthreads();
    if (k0 + BK < K) gload(k0 + BK);
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      frag fa[TM], fb[TN];
      const int ko = kc * KC + (lane >> 4) * EPL;
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[i] = *reinterpret_cast<const frag *>(&As[(wm * (BM / 2) + i * 16 + (lane & 15)) * LDR + ko]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fb[j] = *reinterpret_cast<const frag *>(&Ws[(wn * (BN / 2) + j * 16 + (lane & 15)) * LDR + ko]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = MF::mma(fa[i], fb[j], acc[i][j]);
    }
  }

#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
      epi.tile(m0 + wm * (BM / 2) + i * 16 + 4 * (lane >> 4), n0 + wn * (BN / 2) + j * 16 + (lane & 15),
               acc[i][j], rinv, m0);
}

template <typename T, class Epi>
static void run_gemm(const T *A, int M, int N, int K, const Epi &epi, const GemmPlan &p, hipStream_t s) {
  if (p.skinny) {
    dim3 grid(N / p.nt, p.sk.k_split, (M + 63) / 64);
    switch (p.nt) {
      case 16: hipLaunchKernelGGL((skinny_kernel<T, 16, Epi>), grid, dim3(256), 0, s, A, M, K, epi, p.sk); break;
      case 32: hipLaunchKernelGGL((skinny_kernel<T, 32, Epi>), grid, dim3(256), 0, s, A, M, K, epi, p.sk); break;
      default: hipLaunchKernelGGL((skinny_kernel<T, 64, Epi>), grid, dim3(256), 0, s, A, M, K, epi, p.sk); break;
    }
  } else {
    dim3 grid(N / 64, (M + 63) / 64);
    hipLaunchKernelGGL((tiled_kernel<T, Epi>), grid, dim3(256), 0, s, A, M, K, epi);
  }
}

template <typename T> static void qkv_t(const QkvArgs &a, const GemmPlan &p, hipStream_t s) {
  run_gemm<T>((const T *)a.in.hg, a.M, (a.Hq + 2 * a.Hkv) * a.D, a.in.H, EpiQkv<T>{a}, p, s);
}
template <typename T> static void resid_t(const ResidArgs &a, const GemmPlan &p, hipStream_t s) {
  run_gemm<T>((const T *)a.a, a.M, a.out.H, a.K, EpiResid<T>{a}, p, s);
}
template <typename T> static void swiglu_t(const SwigluArgs &a, const GemmPlan &p, hipStream_t s) {
  run_gemm<T>((const T *)a.in.hg, a.M, 2 * a.F, a.in.H, EpiSwiglu<T>{a}, p, s);
}

int gemm_k_quantum(Dt dt) { return 4 * 4 * (dt == DT_BF16 ? Mfma<bf16>::EPL : Mfma<float>::EPL); }

void launch_qkv(Dt dt, const QkvArgs &a, const GemmPlan &p, hipStream_t s) {
  if (dt == DT_BF16) qkv_t<bf16>(a, p, s); else qkv_t<float>(a, p, s);
}
void launch_resid(Dt dt, const ResidArgs &a, const GemmPlan &p, hipStream_t s) {
  if (dt == DT_BF16) resid_t<bf16>(a, p, s); else resid_t<float>(a, p, s);
}
void launch_swiglu(Dt dt, const SwigluArgs &a, const GemmPlan &p, hipStream_t s) {
  if (dt == DT_BF16) swiglu_t<bf16>(a, p, s); else swiglu_t<float>(a, p, s);
}

}  // namespace dm

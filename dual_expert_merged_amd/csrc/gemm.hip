// Dense projections of the merged layer on gfx950 MFMA: C = A W^T with A token-major
// activations [M][K] and W in the [out][in] layout, fp32 accumulation, fused epilogues:
//   QKV    : RoPE on query/key columns, scatter to query rows and head-major K/V
//   resid  : h += C (fp32 residual stream)
//   swiglu : act = silu(A Wg^T) * (A Wu^T)
// Page "DM0 paper definition vs. Dexbotic code", section 1: each expert applies its own Q/K/V,
// O-projection + residual and MLP; "DM0.5: High-Performance Embodied VLA ...", section 6.3
// names gate/up/down as the MLP GEMMs.
//
// Tiling: a 256-thread workgroup (4 waves as 2x2) owns a BM x BN output tile; each wave a
// (BM/2) x (BN/2) block of 16x16 MFMA tiles.  A and W stream through LDS in 128-byte-per-row
// stages (one 16-byte vector per lane per row chunk, coalesced), prefetched one stage ahead in
// registers.  Column permutations put the two halves of every RoPE pair, and the gate/up pair
// of every SwiGLU column, in lanes l and l^8 of the same MFMA tile so the epilogue combines
// them with one cross-lane exchange.
#include "common.h"
#include "kernels.h"

namespace dm {

__device__ __forceinline__ bool row_valid(const RowMap &rm, int row, int M, int *b_out, int *s_out) {
  if (row >= M) return false;
  const int b = row / rm.rows_per_b, s = row - b * rm.rows_per_b;
  *b_out = b;
  *s_out = s;
  return rm.is_prefix ? (s < min(rm.lens[b], rm.cap)) : true;
}

// Fused Q/K/V: permuted column c of the tile -> global output column of W_qkv.
template <typename T> struct EpiQkv {
  const T *w; int K, M;
  T *q, *k, *v;
  int kv_rows;
  RowMap rows;
  const float2 *rope;
  int Hq, Hkv, D;

  // Within each section (queries, keys, values) the 16-column MFMA tile j carries RoPE pair
  // indices 8j..8j+7: lanes with column < 8 hold element i of the pair, lanes 8..15 element
  // i + D/2 of the same head.
  __device__ __forceinline__ int col(int c) const {
    const int qd = Hq * D, kd = Hkv * D;
    const int base = c < qd ? 0 : (c < qd + kd ? qd : qd + kd);
    const int local = c - base;
    const int half = D >> 1;
    const int p = (local >> 4) * 8 + (local & 7);
    const int upper = (local >> 3) & 1;
    return base + (p / half) * D + (p % half) + upper * half;
  }
  __device__ __forceinline__ const T *wrow(int c) const { return w + (size_t)col(c) * K; }

  __device__ __forceinline__ void tile(int row0, int c, f32x4 acc, int lane) const {
    const int gc = col(c);
    const int qd = Hq * D, kd = Hkv * D;
    const int sec = gc < qd ? 0 : (gc < qd + kd ? 1 : 2);
    const int local = gc - (sec == 0 ? 0 : (sec == 1 ? qd : qd + kd));
    const int head = local / D, d = local - head * D;
    const int half = D >> 1;
    const int upper = d >= half;
    const int i = d - upper * half;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float u = acc[r];
      const float pu = __shfl_xor(u, 8, WAVE);
      int b, s;
      if (!row_valid(rows, row0 + r, M, &b, &s)) continue;
      if (sec < 2) {
        const int pos = rows.is_prefix ? s : max(0, min(rows.lens[b], rows.cap)) + s;
        const float2 cs = rope[(size_t)pos * half + i];
        u = upper ? (u * cs.x + pu * cs.y) : (u * cs.x - pu * cs.y);
      }
      const T val = from_f32<T>(u);
      if (sec == 0) {
        q[(size_t)(row0 + r) * qd + gc] = val;
      } else {
        T *dst = sec == 1 ? k : v;
        dst[((size_t)(b * Hkv + head) * kv_rows + s) * D + d] = val;
      }
    }
  }
};

template <typename T> struct EpiResid {
  const T *w; int K, M, N;
  float *h;
  RowMap rows;
  __device__ __forceinline__ const T *wrow(int c) const { return w + (size_t)c * K; }
  __device__ __forceinline__ void tile(int row0, int c, f32x4 acc, int) const {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int b, s;
      if (!row_valid(rows, row0 + r, M, &b, &s)) continue;
      h[(size_t)(row0 + r) * N + c] += acc[r];
    }
  }
};

// Column c of the tile: MFMA tile j = c/16 carries FFN columns 8j..8j+7, gate in lanes 0..7 and
// up in lanes 8..15.
template <typename T> struct EpiSwiglu {
  const T *wg, *wu; int K, M, F;
  T *act;
  RowMap rows;
  __device__ __forceinline__ const T *wrow(int c) const {
    const int f = (c >> 4) * 8 + (c & 7);
    return ((c >> 3) & 1 ? wu : wg) + (size_t)f * K;
  }
  __device__ __forceinline__ void tile(int row0, int c, f32x4 acc, int) const {
    const int f = (c >> 4) * 8 + (c & 7);
    const int up = (c >> 3) & 1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float g = acc[r];
      const float u = __shfl_xor(g, 8, WAVE);
      int b, s;
      if (up || !row_valid(rows, row0 + r, M, &b, &s)) continue;
      act[(size_t)(row0 + r) * F + f] = from_f32<T>(silu(g) * u);
    }
  }
};

template <typename T, int BM, int BN, class Epi>
__global__ __launch_bounds__(256) void gemm_kernel(const T *__restrict__ A, int M, int K, Epi epi) {
  typedef Mfma<T> MF;
  typedef typename MF::frag frag;
  constexpr int EPL = MF::EPL;
  constexpr int KC = 4 * EPL;           // contraction indices per MFMA k-chunk
  constexpr int BK = 2 * KC;            // per LDS stage: 128 bytes of every row
  constexpr int VPR = BK / EPL;         // 16-byte vectors per row per stage
  constexpr int LDR = BK + EPL;         // padded LDS row, elements
  constexpr int TM = BM / 32, TN = BN / 32;
  constexpr int AV = BM * VPR / 256, WV = BN * VPR / 256;
  static_assert(AV >= 1 && WV >= 1, "tile too small for 256 threads");
  __shared__ __attribute__((aligned(16))) T As[BM * LDR];
  __shared__ __attribute__((aligned(16))) T Ws[BN * LDR];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;

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
               acc[i][j], lane);
}

template <typename T, class Epi>
static void run_gemm(const T *A, int M, int N, int K, const Epi &epi, hipStream_t s) {
  constexpr int BM = 64, BN = 64;
  dim3 grid(N / BN, (M + BM - 1) / BM);
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, Epi>), grid, dim3(256), 0, s, A, M, K, epi);
}

template <typename T> static void qkv_t(const QkvArgs &a, hipStream_t s) {
  EpiQkv<T> e{(const T *)a.w, a.K, a.M, (T *)a.q, (T *)a.k, (T *)a.v, a.kv_rows, a.rows, a.rope,
              a.Hq, a.Hkv, a.D};
  run_gemm<T>((const T *)a.a, a.M, (a.Hq + 2 * a.Hkv) * a.D, a.K, e, s);
}
template <typename T> static void resid_t(const ResidArgs &a, hipStream_t s) {
  EpiResid<T> e{(const T *)a.w, a.K, a.M, a.N, a.h, a.rows};
  run_gemm<T>((const T *)a.a, a.M, a.N, a.K, e, s);
}
template <typename T> static void swiglu_t(const SwigluArgs &a, hipStream_t s) {
  EpiSwiglu<T> e{(const T *)a.wg, (const T *)a.wu, a.K, a.M, a.F, (T *)a.act, a.rows};
  run_gemm<T>((const T *)a.a, a.M, 2 * a.F, a.K, e, s);
}

void launch_qkv(Dt dt, const QkvArgs &a, hipStream_t s) {
  if (dt == DT_BF16) qkv_t<bf16>(a, s); else qkv_t<float>(a, s);
}
void launch_resid(Dt dt, const ResidArgs &a, hipStream_t s) {
  if (dt == DT_BF16) resid_t<bf16>(a, s); else resid_t<float>(a, s);
}
void launch_swiglu(Dt dt, const SwigluArgs &a, hipStream_t s) {
  if (dt == DT_BF16) swiglu_t<bf16>(a, s); else swiglu_t<float>(a, s);
}

}  // namespace dm

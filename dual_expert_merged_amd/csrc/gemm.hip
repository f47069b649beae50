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
//    straight from global memory (16 bytes per lane, the whole slice in flight at once), then
//    reduce through LDS.  Narrow-N GEMMs also split K across workgroups: each writes an fp32 partial
//    tile and a second launch (resid_reduce_kernel) sums them in split order and runs the
//    residual epilogue; the kernel boundary orders the two, so no device-scope fence is needed.
//  * big (bf16, larger M): 128 x 256 (or 128 x 128) per workgroup, double-buffered LDS.
//  * tiled (fp32, larger M): a 64x64 output tile per workgroup, A and W staged through LDS.
// Column permutations put the two halves of every RoPE pair, and the gate/up pair of every
// SwiGLU column, in lanes l and l^8 of one MFMA tile, so one cross-lane exchange joins them.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dm {


// 1/rms of rows m0..m0+rows-1 into inv[], from per-16-column sums of squares: 4 threads per row
// (64 rows per pass of 256 threads), each summing a contiguous quarter of the row's partials with
// all its loads in flight, then a fixed-order exchange.  Rows past M use row M-1 (never read).
__device__ __forceinline__ void rms_prepare(const Hidden &in, int M, float eps, int m0, int rows, float *inv,
                                            const float *row_scale = nullptr) {
  const int nt = in.H >> 4;
  for (int base = 0; base < rows; base += 64) {
    const int t = threadIdx.x, row = base + (t >> 2), part = t & 3;
    const float *p = in.ssq + (size_t)min(m0 + row, M - 1) * nt;
    float s = 0.f;
    if ((nt & 15) == 0) {
      const int per = nt >> 4;  // float4 per thread, at most 16 (H <= 4096)
      const float4 *q4 = reinterpret_cast<const float4 *>(p) + part * per;
      float4 v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = q4[min(j, per - 1)];  // unconditional: loads stay in flight
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j < per) s += (v[j].x + v[j].y) + (v[j].z + v[j].w);
    } else {
      for (int i = part; i < nt; i += 4) s += p[i];
    }
    s = sum4(s);
    const float rs = row_scale ? row_scale[min(m0 + row, M - 1)] : 1.0f;
    if (part == 0) inv[row] = rsqrtf(s / (float)in.H + eps) * rs;
  }
}

// Epilogues run per 16x16 tile in two phases so that their global loads (RoPE table, residual
// rows) are all issued before any is consumed: load() gathers, store() computes and writes.  The
// row facts (sample, token, validity) of a 16-row tile are shared by all its column tiles.
// Rows past M read row M-1 (masked at the store).
struct RowInfo {
  int rc[4];  // row index clamped to M-1
  int b[4], s[4];
  bool ok[4];
  int plen[4];
};
__device__ __forceinline__ RowInfo row_info(const RowMap &rm, int row0, int M) {
  RowInfo ri;
  int len[4];
  // one division for the tile; the 4 consecutive rows step across at most one sample boundary
  const int r0c = min(row0, M - 1);
  const int b0 = r0c / rm.rows_per_b, s0 = r0c - b0 * rm.rows_per_b;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int rc = min(row0 + r, M - 1);
    const int s = s0 + (rc - r0c);
    const int wrap = s >= rm.rows_per_b;
    ri.rc[r] = rc;
    ri.b[r] = b0 + wrap;
    ri.s[r] = s - wrap * rm.rows_per_b;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) len[r] = rm.lens[ri.b[r]];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    ri.plen[r] = max(0, min(len[r], rm.cap));
    ri.ok[r] = (row0 + r < M) && (rm.is_prefix ? ri.s[r] < ri.plen[r] : true);
  }
  return ri;
}

template <typename T> struct EpiQkv {
  QkvArgs a;
  struct St {
    float2 cs[4];
  };
  __device__ __forceinline__ const RowMap &rows() const { return a.rows; }
  // head_dim is a power of two: divisions by D and D/2 are shifts and masks
  __device__ __forceinline__ int dlog() const { return 31 - __builtin_clz(a.D); }
  __device__ __forceinline__ int col(int c) const {
    const int qd = a.Hq * a.D, kd = a.Hkv * a.D;
    const int base = c < qd ? 0 : (c < qd + kd ? qd : qd + kd);
    const int local = c - base;
    const int hl = dlog() - 1, half = a.D >> 1;
    const int p = (local >> 4) * 8 + (local & 7);
    const int upper = (local >> 3) & 1;
    return base + ((p >> hl) << (hl + 1)) + (p & (half - 1)) + upper * half;
  }
  __device__ __forceinline__ const T *wrow(int c) const { return (const T *)a.w + (size_t)col(c) * a.in.H; }
  __device__ __forceinline__ void prepare(int m0, int rows, float *inv) const {
    rms_prepare(a.in, a.M, a.eps, m0, rows, inv);
  }
  __device__ __forceinline__ St load(const RowInfo &ri, int c) const {
    St st;
    const int D = a.D, half = D >> 1;
    const int d = col(c) & (D - 1);
    const int i = d & (half - 1);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pos = a.rows.is_prefix ? ri.s[r] : ri.plen[r] + ri.s[r];
      st.cs[r] = a.rope[(size_t)pos * half + i];  // also read for value columns (unused there)
    }
    return st;
  }
  __device__ __forceinline__ void store(const St &st, const RowInfo &ri, int row0, int c, f32x4 acc, const float *inv,
                                        int m0) const {
    const int gc = col(c);
    const int D = a.D, qd = a.Hq * D, kd = a.Hkv * D;
    const int sec = gc < qd ? 0 : (gc < qd + kd ? 1 : 2);
    const int local = gc - (sec == 0 ? 0 : (sec == 1 ? qd : qd + kd));
    const int head = local >> dlog(), d = local & (D - 1);
    const int upper = d >= (D >> 1);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float u = acc[r] * inv[row0 + r - m0];
      const float pu = lane_xor8(u);
      if (sec < 2) u = upper ? (u * st.cs[r].x + pu * st.cs[r].y) : (u * st.cs[r].x - pu * st.cs[r].y);
      if (!ri.ok[r]) continue;
      const T val = from_f32<T>(u);
      if (sec == 0) {
        ((T *)a.q)[(size_t)(row0 + r) * qd + gc] = val;
      } else {
        T *dst = (T *)(sec == 1 ? a.k : a.v);
        dst[((size_t)(ri.b[r] * a.Hkv + head) * a.kv_rows + ri.s[r]) * D + d] = val;
      }
    }
  }
};

// W: operand type (T, or fp8 with a per-row scale of A and a per-column scale of W).
template <typename T, typename W = T> struct EpiResid {
  static constexpr bool Q = !std::is_same<T, W>::value;
  ResidArgs a;
  struct St {
    float hv[4];
    float gain, s;
  };
  __device__ __forceinline__ const RowMap &rows() const { return a.rows; }
  __device__ __forceinline__ const W *wrow(int c) const { return (const W *)a.w + (size_t)c * a.K; }
  __device__ __forceinline__ void prepare(int m0, int rows, float *inv) const {
    if constexpr (Q)
      for (int t = threadIdx.x; t < rows; t += blockDim.x) inv[t] = a.a_scale[min(m0 + t, a.M - 1)];
  }
  __device__ __forceinline__ St load(const RowInfo &ri, int c) const {
    St st;
#pragma unroll
    for (int r = 0; r < 4; ++r) st.hv[r] = a.out.h[(size_t)ri.rc[r] * a.out.H + c];
    st.gain = a.next_gain ? a.next_gain[c] : 0.f;
    st.s = Q ? a.s_w[c] : 1.0f;
    return st;
  }
  __device__ __forceinline__ void store(const St &st, const RowInfo &ri, int row0, int c, f32x4 acc, const float *inv,
                                        int m0) const {
    const int H = a.out.H;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + r;
      const bool ok = ri.ok[r];
      const float y = Q ? acc[r] * inv[row - m0] * st.s : acc[r];
      const float hn = ok ? st.hv[r] + y : 0.f;
      if (ok) {
        a.out.h[(size_t)row * H + c] = hn;
        if (a.next_gain) ((T *)a.out.hg)[(size_t)row * H + c] = from_f32<T>(hn * st.gain);
      }
      if (a.next_gain) {
        const float sq = sum16(hn * hn);
        if (ok && (c & 15) == 0) a.out.ssq[(size_t)row * (H >> 4) + (c >> 4)] = sq;
      }
    }
  }
};

template <typename T, typename W = T> struct EpiSwiglu {
  static constexpr bool Q = !std::is_same<T, W>::value;
  SwigluArgs a;
  struct St {
    float s;
  };
  __device__ __forceinline__ const RowMap &rows() const { return a.rows; }
  __device__ __forceinline__ const W *wrow(int c) const {
    const int f = (c >> 4) * 8 + (c & 7);
    return (const W *)((c >> 3) & 1 ? a.wu : a.wg) + (size_t)f * a.in.H;
  }
  __device__ __forceinline__ void prepare(int m0, int rows, float *inv) const {
    rms_prepare(a.in, a.M, a.eps, m0, rows, inv, Q ? a.a_scale : nullptr);
  }
  __device__ __forceinline__ St load(const RowInfo &, int c) const {
    St st;
    st.s = 1.0f;
    if constexpr (Q) st.s = ((c >> 3) & 1 ? a.s_up : a.s_gate)[(c >> 4) * 8 + (c & 7)];
    return st;
  }
  __device__ __forceinline__ void store(const St &st, const RowInfo &ri, int row0, int c, f32x4 acc, const float *inv,
                                        int m0) const {
    const int f = (c >> 4) * 8 + (c & 7);
    const int up = (c >> 3) & 1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float g = acc[r] * inv[row0 + r - m0] * st.s;
      const float u = lane_xor8(g);
      if (up || !ri.ok[r]) continue;
      ((T *)a.act)[(size_t)(row0 + r) * a.F + f] = from_f32<T>(silu(g) * u);
    }
  }
};

// ------------------------------------------------------------------------ skinny kernel (M <= 64)
// NK: MFMA k-chunks per wave; every fragment of the workgroup's slice is loaded before the first
// MFMA, so each wave keeps NK*(CT+4) 16-byte loads per lane in flight.
template <typename T, int NT, int NK, class Epi>
__global__ __launch_bounds__(256) void skinny_kernel(const T *__restrict__ A, int M, int K, Epi epi, SplitK sk) {
  typedef Mfma<T> MF;
  typedef typename MF::frag frag;
  constexpr int EPL = MF::EPL, KC = 4 * EPL, CT = NT / 16;
  __shared__ __attribute__((aligned(16))) f32x4 red[4 * 4 * CT * 64];
  __shared__ float rinv[64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int tile = blockIdx.x, split = blockIdx.y, mt = blockIdx.z, m0 = mt * 64;
  const int n0 = tile * NT;
  const int Ks = K / sk.k_split;
  const int k0 = split * Ks + wave * (Ks >> 2);
  const int nrt = min(4, (M - m0 + 15) >> 4);  // row tiles holding valid rows (uniform)

  const T *wp[CT];
#pragma unroll
  for (int j = 0; j < CT; ++j) wp[j] = epi.wrow(n0 + j * 16 + c16) + k0 + g * EPL;
  const T *ap[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) ap[i] = A + (size_t)min(m0 + i * 16 + c16, M - 1) * K + k0 + g * EPL;

  frag wf[NK][CT], af[NK][4];
#pragma unroll
  for (int u = 0; u < NK; ++u)
#pragma unroll
    for (int j = 0; j < CT; ++j) wf[u][j] = load_frag<T>(wp[j] + u * KC);
  // No branch or mask may sit between these loads and their use: a load under a condition, or
  // one whose value is masked right away, is waited for at once and serialises the sequence.
  // Rows past M read row M-1; their outputs are never stored, so they need no mask.
#pragma unroll
  for (int u = 0; u < NK; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) af[u][i] = load_frag<T>(ap[i] + u * KC);

  epi.prepare(m0, 64, rinv);
  // the epilogue's own loads (row lengths, RoPE table, residual rows) go out with the operands
  const RowInfo ri = row_info(epi.rows(), m0 + wave * 16 + 4 * g, M);
  typename Epi::St st[CT];
#pragma unroll
  for (int j = 0; j < CT; ++j) st[j] = epi.load(ri, n0 + j * 16 + c16);

  f32x4 acc[4][CT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < CT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < NK; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < nrt)
#pragma unroll
        for (int j = 0; j < CT; ++j) acc[i][j] = MF::mma(af[u][i], wf[u][j], acc[i][j]);

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
    // K split across workgroups: store this slice's partial sums [split][M][N] (row-major) and
    // leave the sum and the epilogue to resid_reduce_kernel, launched next.
    if (wave < nrt) {
      const int N = gridDim.x * NT;
#pragma unroll
      for (int j = 0; j < CT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + wave * 16 + 4 * g + r;
          if (row < M) sk.part[((size_t)split * M + row) * N + n0 + j * 16 + c16] = sum[j][r];
        }
    }
    return;
  }
  if (wave < nrt) {
#pragma unroll
    for (int j = 0; j < CT; ++j) epi.store(st[j], ri, m0 + wave * 16 + 4 * g, n0 + j * 16 + c16, sum[j], rinv, m0);
  }
}

// Sum of the K-split partials of a residual projection plus the residual epilogue:
// h += sum_s part[s], hg = h * next_gain, per-16-column sums of squares.  Thread = 4 columns of
// one row; the split sum runs in split order.
template <typename T>
__global__ __launch_bounds__(256) void resid_reduce_kernel(ResidArgs a, const float *__restrict__ part, int ks) {
  const int H = a.out.H, q4 = H >> 2;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int row = min(idx / q4, a.M - 1), c = (idx - (idx / q4) * q4) * 4;
  const bool in_range = idx < a.M * q4;
  float4 pv[16];
#pragma unroll
  for (int sp = 0; sp < 16; ++sp)  // unconditional (clamped) loads stay in flight together
    pv[sp] = *reinterpret_cast<const float4 *>(part + ((size_t)min(sp, ks - 1) * a.M + row) * H + c);
  float4 hv = *reinterpret_cast<const float4 *>(a.out.h + (size_t)row * H + c);
  float4 gv = a.next_gain ? *reinterpret_cast<const float4 *>(a.next_gain + c) : make_float4(0.f, 0.f, 0.f, 0.f);
  const int b = row / a.rows.rows_per_b, s = row - b * a.rows.rows_per_b;
  const int plen = max(0, min(a.rows.lens[b], a.rows.cap));
  const bool ok = in_range && (a.rows.is_prefix ? s < plen : true);
  float4 t = pv[0];
#pragma unroll
  for (int sp = 1; sp < 16; ++sp)
    if (sp < ks) {
      t.x += pv[sp].x; t.y += pv[sp].y; t.z += pv[sp].z; t.w += pv[sp].w;
    }
  const float4 hn = make_float4(hv.x + t.x, hv.y + t.y, hv.z + t.z, hv.w + t.w);
  if (ok) {
    *reinterpret_cast<float4 *>(a.out.h + (size_t)row * H + c) = hn;
    if (a.next_gain) {
      T *hg = (T *)a.out.hg + (size_t)row * H + c;
      hg[0] = from_f32<T>(hn.x * gv.x);
      hg[1] = from_f32<T>(hn.y * gv.y);
      hg[2] = from_f32<T>(hn.z * gv.z);
      hg[3] = from_f32<T>(hn.w * gv.w);
    }
  }
  if (a.next_gain) {
    const float sq = sum4(ok ? hn.x * hn.x + hn.y * hn.y + hn.z * hn.z + hn.w * hn.w : 0.f);
    if (ok && (c & 15) == 0) a.out.ssq[(size_t)row * (H >> 4) + (c >> 4)] = sq;
  }
}

// ------------------------------------------------------------------------ big kernel (M > 64)
// Workgroup tile 128 x BN (BN = 256 or 128); four waves as 2 x 2, each 64 x BN/2, i.e. 4 x BN/32
// MFMA 16x16 tiles, so every LDS fragment read feeds several MFMAs.  Each k-step moves 128 bytes
// of every row (64 bf16 or 128 FP8 codes) through two LDS buffers: the next k-step is loaded into
// registers while the current one is multiplied, then stored to the other buffer, one barrier per
// k-step.  Rows are padded to 144 bytes, which spreads the 16 rows of a fragment read over all
// LDS banks.  grid.z splits K (the narrow residual projections), each split writing fp32 partial
// sums for resid_reduce_kernel.  Op: bf16 (two 16x16x32 MFMAs per k-step) or fp8 (one
// 16x16x128 MFMA per k-step).
template <typename Op, int BN, class Epi>
__global__ __launch_bounds__(256) void big_kernel(const Op *__restrict__ A, int M, int K, Epi epi, SplitK sk) {
  constexpr int EB = sizeof(Op);       // bytes per element
  constexpr int BM = 128, RB = 128, LDB = RB + 16;
  constexpr int BK = RB / EB, VE = 16 / EB;
  constexpr int TN = BN / 32;
  constexpr int AV = BM * 8 / 256, WV = BN * 8 / 256;
  __shared__ __attribute__((aligned(16))) char As[2][BM * LDB];
  __shared__ __attribute__((aligned(16))) char Ws[2][BN * LDB];
  __shared__ float rinv[BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM, split = blockIdx.z;
  const int Ks = K / sk.k_split, kb = split * Ks, nkt = Ks / BK;

  const Op *asrc[AV];
  int adst[AV];
#pragma unroll
  for (int v = 0; v < AV; ++v) {
    const int idx = tid + v * 256, r = idx >> 3, cv = idx & 7;
    asrc[v] = A + (size_t)min(m0 + r, M - 1) * K + kb + cv * VE;  // rows past M: never stored
    adst[v] = r * LDB + cv * 16;
  }
  const Op *wsrc[WV];
  int wdst[WV];
#pragma unroll
  for (int v = 0; v < WV; ++v) {
    const int idx = tid + v * 256, r = idx >> 3, cv = idx & 7;
    wsrc[v] = epi.wrow(n0 + r) + kb + cv * VE;
    wdst[v] = r * LDB + cv * 16;
  }
  i32x4 ra[AV], rw[WV];
  auto gload = [&](int kt) {
#pragma unroll
    for (int v = 0; v < AV; ++v) ra[v] = *reinterpret_cast<const i32x4 *>(asrc[v] + kt * BK);
#pragma unroll
    for (int v = 0; v < WV; ++v) rw[v] = *reinterpret_cast<const i32x4 *>(wsrc[v] + kt * BK);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int v = 0; v < AV; ++v) *reinterpret_cast<i32x4 *>(&As[buf][adst[v]]) = ra[v];
#pragma unroll
    for (int v = 0; v < WV; ++v) *reinterpret_cast<i32x4 *>(&Ws[buf][wdst[v]]) = rw[v];
  };

  f32x4 acc[4][TN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  epi.prepare(m0, BM, rinv);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nkt) gload(kt + 1);
    const char *ab = &As[cur][(wm * 64 + c16) * LDB];
    const char *wb = &Ws[cur][(wn * (BN / 2) + c16) * LDB];
    if constexpr (EB == 2) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        bf16x8 fa[4], fb[TN];
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = *reinterpret_cast<const bf16x8 *>(ab + i * 16 * LDB + kc * 64 + g * 16);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[j] = *reinterpret_cast<const bf16x8 *>(wb + j * 16 * LDB + kc * 64 + g * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = Mfma<bf16>::mma(fa[i], fb[j], acc[i][j]);
      }
    } else {
      i32x8 fa[4], fb[TN];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const i32x4 lo = *reinterpret_cast<const i32x4 *>(ab + i * 16 * LDB + g * 32);
        const i32x4 hi = *reinterpret_cast<const i32x4 *>(ab + i * 16 * LDB + g * 32 + 16);
        fa[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const i32x4 lo = *reinterpret_cast<const i32x4 *>(wb + j * 16 * LDB + g * 32);
        const i32x4 hi = *reinterpret_cast<const i32x4 *>(wb + j * 16 * LDB + g * 32 + 16);
        fb[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = Mfma8::mma(fa[i], fb[j], acc[i][j]);
    }
    if (kt + 1 < nkt) lstore(cur ^ 1);
    __syncthreads();
  }

  if (sk.k_split > 1) {  // partial sums [split][M][N], row-major; resid_reduce_kernel finishes
    const int N = gridDim.x * BN;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + wm * 64 + i * 16 + 4 * g + r;
          if (row < M) sk.part[((size_t)split * M + row) * N + n0 + wn * (BN / 2) + j * 16 + c16] = acc[i][j][r];
        }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row0 = m0 + wm * 64 + i * 16 + 4 * g;
    if (row0 - 4 * g >= M) break;  // uniform over the wave: the whole 16-row tile is past M
    const RowInfo ri = row_info(epi.rows(), row0, M);
    typename Epi::St st[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) st[j] = epi.load(ri, n0 + wn * (BN / 2) + j * 16 + c16);
#pragma unroll
    for (int j = 0; j < TN; ++j) epi.store(st[j], ri, row0, n0 + wn * (BN / 2) + j * 16 + c16, acc[i][j], rinv, m0);
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

  const T *asrc[AV];  // rows past M read row M-1: their outputs are never stored
  int adst[AV];
#pragma unroll
  for (int v = 0; v < AV; ++v) {
    const int idx = tid + v * 256, r = idx / VPR, cv = idx % VPR;
    asrc[v] = A + (size_t)min(m0 + r, M - 1) * K + cv * EPL;
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
    for (int v = 0; v < AV; ++v) ra[v] = load_frag<T>(asrc[v] + k0);
#pragma unroll
    for (int v = 0; v < WV; ++v) rw[v] = load_frag<T>(wsrc[v] + k0);
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  epi.prepare(m0, 64, rinv);
  RowInfo ri[TM];
  typename Epi::St st[TM][TN];  // the epilogue's loads go out with the first operand tiles
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    ri[i] = row_info(epi.rows(), m0 + wm * (BM / 2) + i * 16 + 4 * (lane >> 4), M);
#pragma unroll
    for (int j = 0; j < TN; ++j) st[i][j] = epi.load(ri[i], n0 + wn * (BN / 2) + j * 16 + (lane & 15));
  }
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
      epi.store(st[i][j], ri[i], m0 + wm * (BM / 2) + i * 16 + 4 * (lane >> 4),
                n0 + wn * (BN / 2) + j * 16 + (lane & 15), acc[i][j], rinv, m0);
}

template <typename T, int NT, class Epi>
static void run_skinny(const T *A, int M, int N, int K, const Epi &epi, const GemmPlan &p, hipStream_t s) {
  dim3 grid(N / NT, p.sk.k_split, (M + 63) / 64);
  const int nk = K / p.sk.k_split / 4 / (4 * Mfma<T>::EPL);
  switch (nk) {
#define DM_NK(n) case n: hipLaunchKernelGGL((skinny_kernel<T, NT, n, Epi>), grid, dim3(256), 0, s, A, M, K, epi, p.sk); break;
    DM_NK(1) DM_NK(2) DM_NK(3) DM_NK(4) DM_NK(5) DM_NK(6) DM_NK(7) DM_NK(8)
#undef DM_NK
    default: break;  // the host plan never asks for more than 8 k-chunks per wave
  }
}

template <typename T, class Epi>
static void run_gemm(const T *A, int M, int N, int K, const Epi &epi, const GemmPlan &p, hipStream_t s) {
  if (p.skinny) {
    switch (p.nt) {
      case 16: run_skinny<T, 16>(A, M, N, K, epi, p, s); break;
      case 32: run_skinny<T, 32>(A, M, N, K, epi, p, s); break;
      default: run_skinny<T, 64>(A, M, N, K, epi, p, s); break;
    }
  } else if (p.nt >= 128) {
    if constexpr (std::is_same<T, bf16>::value) {
      dim3 grid(N / p.nt, (M + 127) / 128, p.sk.k_split);
      if (p.nt == 256)
        hipLaunchKernelGGL((big_kernel<bf16, 256, Epi>), grid, dim3(256), 0, s, A, M, K, epi, p.sk);
      else
        hipLaunchKernelGGL((big_kernel<bf16, 128, Epi>), grid, dim3(256), 0, s, A, M, K, epi, p.sk);
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
  if (p.sk.k_split > 1) {
    const int n = a.M * (a.out.H / 4);
    hipLaunchKernelGGL(resid_reduce_kernel<T>, dim3((n + 255) / 256), dim3(256), 0, s, a, p.sk.part, p.sk.k_split);
  }
}
template <typename T> static void swiglu_t(const SwigluArgs &a, const GemmPlan &p, hipStream_t s) {
  run_gemm<T>((const T *)a.in.hg, a.M, 2 * a.F, a.in.H, EpiSwiglu<T>{a}, p, s);
}

// FP8: one launch of the large-tile kernel, 256 columns per workgroup when N allows it.
template <class Epi> static void run_fp8(const fp8 *A, int M, int N, int K, const Epi &epi, hipStream_t s) {
  const SplitK none{1, nullptr};
  if (N % 256 == 0)
    hipLaunchKernelGGL((big_kernel<fp8, 256, Epi>), dim3(N / 256, (M + 127) / 128), dim3(256), 0, s, A, M, K, epi, none);
  else
    hipLaunchKernelGGL((big_kernel<fp8, 128, Epi>), dim3(N / 128, (M + 127) / 128), dim3(256), 0, s, A, M, K, epi, none);
}
void launch_resid_fp8(const ResidArgs &a, hipStream_t s) {
  run_fp8((const fp8 *)a.a, a.M, a.out.H, a.K, EpiResid<bf16, fp8>{a}, s);
}
void launch_swiglu_fp8(const SwigluArgs &a, hipStream_t s) {
  run_fp8((const fp8 *)a.a8, a.M, 2 * a.F, a.in.H, EpiSwiglu<bf16, fp8>{a}, s);
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

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
// Three kernels share the epilogues:
//  * skinny (few rows: the action chunk of one or two samples): one workgroup owns NT output
//    columns for 64 (or 32 / 16) rows and one K slice, more rows taking more row blocks; its 4 waves each take a quarter of the slice and load MFMA fragments
//    straight from global memory (16 bytes per lane, the whole slice in flight at once), then
//    reduce through LDS.  Narrow-N GEMMs also split K across workgroups: each writes an fp32 partial
//    tile and a second launch (resid_reduce_kernel) sums them in split order and runs the
//    residual epilogue; the kernel boundary orders the two, so no device-scope fence is needed.
//  * big (bf16 or FP8, larger M): 128 x 128, 128 x 256 or 128 x 384 per workgroup, operands
//    copied global -> LDS with two (or one) k-steps in flight.
//  * tiled (fp32, larger M): a 64x64 output tile per workgroup, A and W staged through LDS.
// Column permutations put the two halves of every RoPE pair, and the gate/up pair of every
// SwiGLU column, in the same lane of two adjacent 16-column MFMA tiles, so each lane joins them
// with no cross-lane exchange.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dm {


// 1/rms of rows m0..m0+rows-1 into inv[], from per-16-column sums of squares: 4 threads per row
// (64 rows per pass of 256 threads), each summing a contiguous quarter of the row's partials with
// all its loads in flight, then a fixed-order exchange.  Rows past M use row M-1 (never read).
__device__ __forceinline__ void rms_prepare(const Hidden &in, int M, float eps, int m0, int rows, float *inv,
                                            const float *row_scale = nullptr) {
  if (!in.ssq) {  // operand already normalised (time-modulated norm): only the row scale
    for (int t = threadIdx.x; t < rows; t += blockDim.x) inv[t] = row_scale ? row_scale[min(m0 + t, M - 1)] : 1.0f;
    return;
  }
  const int nt = in.H >> 4;
  const int step = blockDim.x >> 2;  // rows per pass
  for (int base = 0; base < rows; base += step) {
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
    if (part == 0 && row < rows) inv[row] = rsqrtf(s / (float)in.H + eps) * rs;
  }
}

// The same for the 64 rows of the skinny kernel in two steps: rms_load issues the loads of the
// sums of squares, rms_finish reduces them once they have arrived, so the operand loads can be
// issued in between (loads complete in issue order: these small ones first).
struct RmsPre {
  float4 v[16];
};
__device__ __forceinline__ RmsPre rms_load(const Hidden &in, int M, int m0) {
  RmsPre p;
  const int nt = in.H >> 4, t = threadIdx.x, row = t >> 2, part = t & 3;
  if (in.ssq && (nt & 15) == 0) {
    const int per = nt >> 4;
    const float4 *q4 = reinterpret_cast<const float4 *>(in.ssq + (size_t)min(m0 + row, M - 1) * nt) + part * per;
#pragma unroll
    for (int j = 0; j < 16; ++j) p.v[j] = q4[min(j, per - 1)];
  }
  return p;
}
__device__ __forceinline__ void rms_finish(const RmsPre &p, const Hidden &in, int M, float eps, int m0, float *inv,
                                           const float *row_scale = nullptr) {
  const int nt = in.H >> 4, t = threadIdx.x, row = t >> 2, part = t & 3;
  if (!in.ssq) {  // operand already normalised (time-modulated norm): only the row scale
    if (part == 0 && row < 64) inv[row] = row_scale ? row_scale[min(m0 + row, M - 1)] : 1.0f;
    return;
  }
  float s = 0.f;
  if ((nt & 15) == 0) {
    const int per = nt >> 4;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < per) s += (p.v[j].x + p.v[j].y) + (p.v[j].z + p.v[j].w);
  } else {
    const float *q = in.ssq + (size_t)min(m0 + row, M - 1) * nt;
    for (int i = part; i < nt; i += 4) s += q[i];
  }
  s = sum4(s);
  const float rs = row_scale ? row_scale[min(m0 + row, M - 1)] : 1.0f;
  if (part == 0 && row < 64) inv[row] = rsqrtf(s / (float)in.H + eps) * rs;
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
  // one division for the tile when a sample has at least 4 rows (the 4 consecutive rows then
  // step across at most one sample boundary); otherwise one per row
  const int r0c = min(row0, M - 1);
  const int b0 = r0c / rm.rows_per_b, s0 = r0c - b0 * rm.rows_per_b;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int rc = min(row0 + r, M - 1);
    ri.rc[r] = rc;
    if (rm.rows_per_b >= 4) {  // uniform
      const int s = s0 + (rc - r0c);
      const int wrap = s >= rm.rows_per_b;
      ri.b[r] = b0 + wrap;
      ri.s[r] = s - wrap * rm.rows_per_b;
    } else {
      ri.b[r] = rc / rm.rows_per_b;
      ri.s[r] = rc - ri.b[r] * rm.rows_per_b;
    }
  }
  if (rm.is_prefix) {  // uniform; action rows need no prefix length (their RoPE rows are precomputed)
#pragma unroll
    for (int r = 0; r < 4; ++r) len[r] = rm.lens[ri.b[r]];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ri.plen[r] = max(0, min(len[r], rm.cap));
      ri.ok[r] = (row0 + r < M) && ri.s[r] < ri.plen[r];
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ri.plen[r] = 0;
      ri.ok[r] = row0 + r < M;
    }
  }
  return ri;
}

template <typename T> struct EpiQkv {
  QkvArgs a;
  struct St {
    float2 cs[4];
  };
  __device__ __forceinline__ const RowMap &rows() const { return a.rows; }
  // head_dim is a power of two: divisions by D are shifts and masks
  __device__ __forceinline__ int dlog() const { return 31 - __builtin_clz(a.D); }
  // Column permutation: the 16-column tiles of a head come in pairs (2p, 2p+1) holding dims
  // p*16 + l and D/2 + p*16 + l, so the two halves of every rotate-half RoPE pair sit in one lane.
  __device__ __forceinline__ int col(int c) const {
    const int qd = a.Hq * a.D, kd = a.Hkv * a.D;
    const int base = c < qd ? 0 : (c < qd + kd ? qd : qd + kd);
    const int local = c - base, dl = dlog();
    const int t = (local & (a.D - 1)) >> 4;
    return base + ((local >> dl) << dl) + (t & 1) * (a.D >> 1) + (t >> 1) * 16 + (local & 15);
  }
  __device__ __forceinline__ const T *wrow(int c) const { return (const T *)a.w + (size_t)col(c) * a.in.H; }
  __device__ __forceinline__ void prepare(int m0, int rows, float *inv) const {
    rms_prepare(a.in, a.M, a.eps, m0, rows, inv);
  }
  typedef RmsPre Pre;
  __device__ __forceinline__ Pre pre_load(int m0) const { return rms_load(a.in, a.M, m0); }
  __device__ __forceinline__ void pre_finish(const Pre &p, int m0, float *inv) const {
    rms_finish(p, a.in, a.M, a.eps, m0, inv);
  }
  // (cos, sin) of the row's position for the even tile of a pair (the odd tile shares them):
  // prefix token s at s (table by position), action rows from the per-row table (position
  // P_b + s, filled once per call)
  __device__ __forceinline__ St load(const RowInfo &ri, int c) const {
    St st;
    if ((c >> 4) & 1) return st;  // uniform per tile
    const int i = col(c) & ((a.D >> 1) - 1);
#pragma unroll
    for (int r = 0; r < 4; ++r)  // also read for value columns (unused there): a branch here
      // would make the compiler wait for each load where it is issued
      st.cs[r] = a.rows.is_prefix ? a.rope[(size_t)ri.s[r] * (a.D >> 1) + i] : a.rope_rows[(size_t)ri.rc[r] * (a.D >> 1) + i];
    return st;
  }
  // rotate-half RoPE of the lane's pair (lo = dim d, hi = dim d + D/2) for rows of the q and k
  // sections; v passes through
  __device__ __forceinline__ void rotate(const St &st, int gc, float &lo, float &hi, int r) const {
    if (a.q_norm) return;  // QK-norm first: qk_norm_rope_kernel rotates after normalising
    if (gc < (a.Hq + a.Hkv) * a.D) {
      const float l = lo, h = hi;
      lo = l * st.cs[r].x - h * st.cs[r].y;
      hi = h * st.cs[r].x + l * st.cs[r].y;
    }
  }
  // Large tiles: a 128 x 256 tile is two whole heads of one section (q, k or v).  to_lds2 puts
  // the rotated values at their natural (head, d) position of row (row - m0) of the staging tile;
  // lds_out then writes each row's two heads as whole 16-byte vectors.
  static constexpr bool kTile = true;
  // every tile must lie inside one section: q, k and v widths are multiples of the tile width
  __device__ __forceinline__ bool tile_ok(int bn) const { return (a.Hq * a.D) % bn == 0 && (a.Hkv * a.D) % bn == 0; }
  template <class Tile>
  __device__ __forceinline__ void to_lds2(const St &st, const St &, int row0, int c, f32x4 acc0, f32x4 acc1,
                                          const float *inv, int m0, int n0, const Tile &ot) const {
    const int gc = col(c), local = gc - col(n0);  // (head - first head) * D + d of the low half
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float lo = acc0[r] * inv[row0 + r - m0], hi = acc1[r] * inv[row0 + r - m0];
      rotate(st, gc, lo, hi, r);
      T *orow = ot.row(row0 + r - m0);
      orow[local] = from_f32<T>(lo);
      orow[local + (a.D >> 1)] = from_f32<T>(hi);
    }
  }
  template <int BM, int BN, class Tile>
  __device__ __forceinline__ void lds_out(const Tile &ot, int m0, int n0, int M) const {
    constexpr int CPR = BN / 8;  // 16-byte chunks per row
    const int D = a.D, qd = a.Hq * D, kd = a.Hkv * D;
    const int gc0 = col(n0);
    const int sec = gc0 < qd ? 0 : (gc0 < qd + kd ? 1 : 2);
    const int head0 = (gc0 - (sec == 0 ? 0 : (sec == 1 ? qd : qd + kd))) >> dlog();
    const RowMap &rm = a.rows;
#pragma unroll 4
    for (int idx = threadIdx.x; idx < BM * CPR; idx += blockDim.x) {
      const int rl = idx / CPR, ch = idx - rl * CPR, row = m0 + rl;
      if (row >= M) continue;
      const int b = row / rm.rows_per_b, s = row - b * rm.rows_per_b;
      if (rm.is_prefix && s >= max(0, min(rm.lens[b], rm.cap))) continue;
      const i32x4 v = *reinterpret_cast<const i32x4 *>(ot.row(rl) + ch * 8);
      T *dst;
      if (sec == 0) {
        dst = (T *)a.q + (size_t)row * qd + gc0 + ch * 8;
      } else {
        const int hl = (ch * 8) >> dlog(), d = ch * 8 - (hl << dlog());
        dst = (T *)(sec == 1 ? a.k : a.v) + ((size_t)(b * a.Hkv + head0 + hl) * a.kv_rows + s) * D + d;
      }
      *reinterpret_cast<i32x4 *>(dst) = v;
    }
  }
  // tile pair (c, c + 16): the low and high halves of 16 RoPE pairs
  __device__ __forceinline__ void store2(const St &st, const St &, const RowInfo &ri, int row0, int c, f32x4 acc0,
                                         f32x4 acc1, bool, const float *inv, int m0) const {
    const int gc = col(c);
    const int D = a.D, qd = a.Hq * D, kd = a.Hkv * D;
    const int sec = gc < qd ? 0 : (gc < qd + kd ? 1 : 2);
    const int local = gc - (sec == 0 ? 0 : (sec == 1 ? qd : qd + kd));
    const int head = local >> dlog(), d = local & (D - 1);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float lo = acc0[r] * inv[row0 + r - m0], hi = acc1[r] * inv[row0 + r - m0];
      rotate(st, gc, lo, hi, r);
      if (!ri.ok[r]) continue;
      T *dst = sec == 0 ? (T *)a.q + (size_t)(row0 + r) * qd + gc
                        : (T *)(sec == 1 ? a.k : a.v) + ((size_t)(ri.b[r] * a.Hkv + head) * a.kv_rows + ri.s[r]) * D + d;
      dst[0] = from_f32<T>(lo);
      dst[D >> 1] = from_f32<T>(hi);
    }
  }
};

// W: operand type (T, or fp8 with a per-row scale of A and a per-column scale of W).
template <typename T, typename W = T> struct EpiResid {
  static constexpr bool Q = !std::is_same<T, W>::value;
  ResidArgs a;
  struct St {
    float hv[4];
    float gain, s, gate;
  };
  __device__ __forceinline__ const RowMap &rows() const { return a.rows; }
  __device__ __forceinline__ const W *wrow(int c) const { return (const W *)a.w + (size_t)c * a.K; }
  __device__ __forceinline__ void prepare(int m0, int rows, float *inv) const {
    if constexpr (Q)
      for (int t = threadIdx.x; t < rows; t += blockDim.x) inv[t] = a.a_scale[min(m0 + t, a.M - 1)];
  }
  static constexpr bool kTile = false;
  __device__ __forceinline__ bool tile_ok(int) const { return false; }
  template <class Tile>
  __device__ __forceinline__ void to_lds2(const St &, const St &, int, int, f32x4, f32x4, const float *, int, int,
                                          const Tile &) const {}
  template <int BM, int BN, class Tile>
  __device__ __forceinline__ void lds_out(const Tile &, int, int, int) const {}
  struct Pre {};
  __device__ __forceinline__ Pre pre_load(int) const { return Pre{}; }
  __device__ __forceinline__ void pre_finish(const Pre &, int m0, float *inv) const { prepare(m0, 64, inv); }
  __device__ __forceinline__ St load(const RowInfo &ri, int c) const {
    St st;
#pragma unroll
    for (int r = 0; r < 4; ++r) st.hv[r] = a.out.h[(size_t)ri.rc[r] * a.out.H + c];
    st.gain = a.next_gain ? a.next_gain[c] : 0.f;
    st.s = Q ? a.s_w[c] : 1.0f;
    st.gate = a.gate ? a.gate[c] : 1.0f;
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
      const float hn = ok ? st.hv[r] + (a.gate ? st.gate * y : y) : 0.f;
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
  __device__ __forceinline__ void store2(const St &st0, const St &st1, const RowInfo &ri, int row0, int c, f32x4 acc0,
                                         f32x4 acc1, bool has1, const float *inv, int m0) const {
    store(st0, ri, row0, c, acc0, inv, m0);
    if (has1) store(st1, ri, row0, c + 16, acc1, inv, m0);
  }
};

template <typename T, typename W = T> struct EpiSwiglu {
  static constexpr bool Q = !std::is_same<T, W>::value;
  SwigluArgs a;
  struct St {
    float s;
  };
  __device__ __forceinline__ const RowMap &rows() const { return a.rows; }
  // Column permutation: 16-column tiles come in pairs (2q, 2q+1) = gate and up rows of the same
  // 16 activation columns f = 16q + l, so silu(gate) * up is formed within one lane.
  __device__ __forceinline__ static int act_col(int c) { return (c >> 5) * 16 + (c & 15); }
  __device__ __forceinline__ const W *wrow(int c) const {
    return (const W *)((c >> 4) & 1 ? a.wu : a.wg) + (size_t)act_col(c) * a.in.H;
  }
  __device__ __forceinline__ void prepare(int m0, int rows, float *inv) const {
    rms_prepare(a.in, a.M, a.eps, m0, rows, inv, Q ? a.a_scale : nullptr);
  }
  typedef RmsPre Pre;
  __device__ __forceinline__ Pre pre_load(int m0) const { return rms_load(a.in, a.M, m0); }
  __device__ __forceinline__ void pre_finish(const Pre &p, int m0, float *inv) const {
    rms_finish(p, a.in, a.M, a.eps, m0, inv, Q ? a.a_scale : nullptr);
  }
  __device__ __forceinline__ St load(const RowInfo &, int c) const {
    St st;
    st.s = 1.0f;
    if constexpr (Q) st.s = ((c >> 4) & 1 ? a.s_up : a.s_gate)[act_col(c)];
    return st;
  }
  // Large tiles: the 2*16 columns of a tile pair are 16 activation columns; to_lds2 stages them
  // per row, lds_out writes each row's BN/2 values as whole 16-byte vectors.
  static constexpr bool kTile = true;
  __device__ __forceinline__ bool tile_ok(int) const { return true; }
  template <class Tile>
  __device__ __forceinline__ void to_lds2(const St &sg, const St &su, int row0, int c, f32x4 accg, f32x4 accu,
                                          const float *inv, int m0, int n0, const Tile &ot) const {
    const int fl = act_col(c) - (n0 >> 1);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float sc = inv[row0 + r - m0];
      ot.row(row0 + r - m0)[fl] = from_f32<T>(silu(accg[r] * sc * sg.s) * (accu[r] * sc * su.s));
    }
  }
  template <int BM, int BN, class Tile>
  __device__ __forceinline__ void lds_out(const Tile &ot, int m0, int n0, int M) const {
    constexpr int CPR = BN / 16;  // 16-byte chunks of activation per row
    const RowMap &rm = a.rows;
#pragma unroll 4
    for (int idx = threadIdx.x; idx < BM * CPR; idx += blockDim.x) {
      const int rl = idx / CPR, ch = idx - rl * CPR, row = m0 + rl;
      if (row >= M) continue;
      if (rm.is_prefix) {
        const int b = row / rm.rows_per_b, s = row - b * rm.rows_per_b;
        if (s >= max(0, min(rm.lens[b], rm.cap))) continue;
      }
      *reinterpret_cast<i32x4 *>((T *)a.act + (size_t)row * a.F + (n0 >> 1) + ch * 8) =
          *reinterpret_cast<const i32x4 *>(ot.row(rl) + ch * 8);
    }
  }
  __device__ __forceinline__ void store2(const St &sg, const St &su, const RowInfo &ri, int row0, int c, f32x4 accg,
                                         f32x4 accu, bool, const float *inv, int m0) const {
    const int f = act_col(c);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (!ri.ok[r]) continue;
      const float sc = inv[row0 + r - m0];
      ((T *)a.act)[(size_t)(row0 + r) * a.F + f] = from_f32<T>(silu(accg[r] * sc * sg.s) * (accu[r] * sc * su.s));
    }
  }
};

// ------------------------------------------------------------------------ skinny kernel (few rows)
// NK: MFMA k-chunks per wave; every fragment of the workgroup's slice is loaded before the first
// MFMA, so each wave keeps NK*(CT+RT) 16-byte loads per lane in flight.
// RT: 16-row tiles per workgroup (4, or 2 / 1 to spread a narrow GEMM over more workgroups,
// each reading fewer activation rows).
// NWV: waves per workgroup, each taking 1/NWV of the K slice (4; 16 lets one workgroup cover a
// residual projection's whole K with all its loads in flight, so no split and no second launch).
template <typename T, int NT, int NK, int RT, int NWV, class Epi>
__global__ __launch_bounds__(NWV * 64) void skinny_kernel(const T *__restrict__ A, int M, int K, Epi epi, SplitK sk) {
  typedef Mfma<T> MF;
  typedef typename MF::frag frag;
  constexpr int EPL = MF::EPL, KC = 4 * EPL, CT = NT / 16;
  static_assert(RT == 1 || RT == 2 || RT == 4, "1, 2 or 4 row tiles");
  __shared__ __attribute__((aligned(16))) f32x4 red[NWV * RT * CT * 64];
  __shared__ float rinv[64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int tile = blockIdx.x, split = blockIdx.y, mt = blockIdx.z, m0 = mt * (16 * RT);
  const int n0 = tile * NT;
  const int Ks = K / sk.k_split;
  const int k0 = split * Ks + wave * (Ks / NWV);
  const int nrt = min(RT, (M - m0 + 15) >> 4);  // row tiles holding valid rows (uniform)

  const T *wp[CT];
#pragma unroll
  for (int j = 0; j < CT; ++j) wp[j] = epi.wrow(n0 + j * 16 + c16) + k0 + g * EPL;
  const T *ap[RT];
#pragma unroll
  for (int i = 0; i < RT; ++i) ap[i] = A + (size_t)min(m0 + i * 16 + c16, M - 1) * K + k0 + g * EPL;

  // The small loads go first (norm statistics, row facts, RoPE / residual rows): loads complete
  // in issue order, so their consumers run while the operand loads below are still in flight.
  const typename Epi::Pre pre = epi.pre_load(m0);
  const RowInfo ri = row_info(epi.rows(), m0 + wave * 16 + 4 * g, M);
  typename Epi::St st[CT];
#pragma unroll
  for (int j = 0; j < CT; ++j) st[j] = epi.load(ri, n0 + j * 16 + c16);

  frag wf[NK][CT], af[NK][RT];
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
    for (int i = 0; i < RT; ++i) af[u][i] = load_frag<T>(ap[i] + u * KC);

  epi.pre_finish(pre, m0, rinv);

  f32x4 acc[RT][CT];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < CT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < NK; ++u)
#pragma unroll
    for (int i = 0; i < RT; ++i)
      if (i < nrt)
#pragma unroll
        for (int j = 0; j < CT; ++j) acc[i][j] = MF::mma(af[u][i], wf[u][j], acc[i][j]);

#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < CT; ++j) red[((wave * RT + i) * CT + j) * 64 + lane] = acc[i][j];
  __syncthreads();
  // wave w < RT sums row tile w over the NWV K slices; the other waves are done (no barrier
  // follows)
  if (wave >= nrt) return;
  f32x4 sum[CT];
#pragma unroll
  for (int j = 0; j < CT; ++j) {
    f32x4 t = red[((0 * RT + wave) * CT + j) * 64 + lane];
#pragma unroll
    for (int w = 1; w < NWV; ++w) t += red[((w * RT + wave) * CT + j) * 64 + lane];
    sum[j] = t;
  }

  if (sk.k_split > 1) {
    // K split across workgroups: store this slice's partial sums [split][M][N] (row-major) and
    // leave the sum and the epilogue to resid_reduce_kernel, launched next.
    const int N = gridDim.x * NT;
#pragma unroll
    for (int j = 0; j < CT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wave * 16 + 4 * g + r;
        if (row < M) sk.part[((size_t)split * M + row) * N + n0 + j * 16 + c16] = sum[j][r];
      }
    return;
  }
#pragma unroll
  for (int j = 0; j < CT; j += 2) {
    const int j1 = j + 1 < CT ? j + 1 : j;
    epi.store2(st[j], st[j1], ri, m0 + wave * 16 + 4 * g, n0 + j * 16 + c16, sum[j], sum[j1], j + 1 < CT, rinv, m0);
  }
}

// Sum of the K-split partials of a residual projection plus the residual epilogue:
// h += sum_s part[s] (times gate when set), hg = h * next_gain, per-16-column sums of squares.  Thread = 4 columns of
// one row; the split sum runs in split order.  KS: the number of splits (all its loads in flight).
template <typename T, int KS>
__global__ __launch_bounds__(256) void resid_reduce_kernel(ResidArgs a, const float *__restrict__ part) {
  const int H = a.out.H, q4 = H >> 2;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int row = min(idx / q4, a.M - 1), c = (idx - (idx / q4) * q4) * 4;
  const bool in_range = idx < a.M * q4;
  float4 pv[KS];
#pragma unroll
  for (int sp = 0; sp < KS; ++sp)
    pv[sp] = *reinterpret_cast<const float4 *>(part + ((size_t)sp * a.M + row) * H + c);
  float4 hv = *reinterpret_cast<const float4 *>(a.out.h + (size_t)row * H + c);
  float4 gv = a.next_gain ? *reinterpret_cast<const float4 *>(a.next_gain + c) : make_float4(0.f, 0.f, 0.f, 0.f);
  const float4 gt = a.gate ? *reinterpret_cast<const float4 *>(a.gate + c) : make_float4(1.f, 1.f, 1.f, 1.f);
  bool ok = in_range;
  if (a.rows.is_prefix) {  // uniform: action rows need no prefix length
    const int b = row / a.rows.rows_per_b, s = row - b * a.rows.rows_per_b;
    ok = ok && s < max(0, min(a.rows.lens[b], a.rows.cap));
  }
  float4 t = pv[0];
#pragma unroll
  for (int sp = 1; sp < KS; ++sp) {
    t.x += pv[sp].x; t.y += pv[sp].y; t.z += pv[sp].z; t.w += pv[sp].w;
  }
  if (a.gate) t = make_float4(gt.x * t.x, gt.y * t.y, gt.z * t.z, gt.w * t.w);
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
// Workgroup tile 128 x BN (BN = 128, 256 or 384), 256 x 256 or 64 x 128; NW waves as WM x WN (8 as 2 x 4,
// or 4 x 2 for 256 rows), each (BM/WM) x (BN/WN), i.e. several MFMA 16x16 tiles, so every LDS
// fragment read feeds several MFMAs, and several waves per SIMD (one LDS-bound workgroup per
// CU) hide each other's LDS and barrier waits.  Each k-step moves 128 bytes of every row (64
// bf16 or 128 FP8 codes).  Operands go from global memory straight into LDS
// (global_load_lds_dwordx4: no registers, whole 128-byte lines per row) through NBUF stage
// buffers (3; 4 for the 192-row stages of the 128 x 64 tile; 2 for the 512-row stages of the
// 128 x 384 and 256 x 256 tiles): while step k is multiplied, the next NBUF-1 steps are loading.  The stage buffers are distinct LDS arrays
// and the k-loop is unrolled by NBUF, so the compiler can tell that reading one buffer does not
// wait for the loads into another, and it interleaves the fragment reads with the MFMAs.  An
// LDS row holds its eight 16-byte chunks in XOR-swizzled order (chunk c at position
// c ^ (row & 7)), so the 16 rows of a fragment read spread over all banks.  grid.z splits K
// (the narrow residual projections), each split writing fp32 partial sums for
// resid_reduce_kernel.  Workgroups are numbered so that the tiles sharing an operand column run
// on the same XCD (blocks go to the 8 XCDs round-robin) and meet in its L2.  Op: bf16 (two
// 16x16x32 MFMAs per k-step) or fp8 (one 16x16x128 MFMA per k-step).

// The finished tile staged in LDS before the coalesced stores: rows 0..63 in one stage buffer,
// 64..127 in another, LD elements per row.
template <typename T, int LD> struct TileRows {
  T *lo, *hi;
  __device__ __forceinline__ T *row(int r) const { return (r < 64 ? lo : hi) + (r & 63) * LD; }
};

// The k-step buffers, one LDS array per buffer and stage size, named statically by the k-step
// code (only the ones a kernel uses are allocated).
template <int SZ, int I> __shared__ __attribute__((aligned(1024))) char big_sb[SZ];
template <int SZ, int B> __device__ __forceinline__ char *big_buf() { return big_sb<SZ, B>; }

template <int I, int N, class F> __device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// NW waves as WM x (NW / WM), each (BM / WM) x (BN * WM / NW); BM = 128 or 256 rows of A
template <typename Op, int BN, int NBUF, int NW, int WM, int BM, class Epi>
__global__ __launch_bounds__(NW * 64) void big_kernel(const Op *__restrict__ A, int M, int K, Epi epi, SplitK sk, int n_tiles,
                                                  int m_tiles, int group_m) {
  constexpr int EB = sizeof(Op);       // bytes per element
  constexpr int RB = 128;              // bytes per row per k-step
  constexpr int BK = RB / EB, VE = 16 / EB;
  constexpr int WN = NW / WM, TN = BN / (16 * WN);  // waves along N, 16-column tiles per wave
  constexpr int TM = BM / (16 * WM);                // 16-row tiles per wave
  constexpr int ROWS = BM + BN;                 // LDS rows per stage (A then W)
  constexpr int LPW = ROWS * RB / 1024 / NW;    // 1 KB DMA instructions per wave per stage
  static_assert(TN % 2 == 0 && LPW * NW * 1024 == ROWS * RB, "wave tiling");
  constexpr int STAGE = ROWS * RB;
  static_assert(NBUF >= 2 && NBUF <= 4, "two to four k-step buffers");
  static_assert(NBUF * STAGE + BM * 4 <= 160 * 1024, "buffers fit the LDS");
  __shared__ float rinv[BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int wm = wave / WN, wn = wave % WN;
  // XCD-aware tile order: the blocks on one XCD (b % 8) take a contiguous run of tiles, ordered
  // in bands of group_m row tiles (uniform, chosen by the host): m fastest within a band, then n,
  // then the next band, the K split outermost (group_m = m_tiles: m fastest; 1: n fastest)
  const int T = n_tiles * m_tiles * (int)gridDim.z;
  const int b = blockIdx.x + (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x;
  const int xcd = b & 7, per = T >> 3, rem = T & 7;
  const int t = xcd * per + min(xcd, rem) + (b >> 3);
  const int mn = m_tiles * n_tiles, split = t / mn, r = t - split * mn;
  const int band = r / (group_m * n_tiles), gm = min(group_m, m_tiles - band * group_m);
  const int local = r - band * group_m * n_tiles;
  const int m_t = band * group_m + local % gm, n_t = local / gm;
  const int n0 = n_t * BN, m0 = m_t * BM;
  const int Ks = K / sk.k_split, kb = split * Ks, nkt = Ks / BK;
  // Tiles that share an operand row run on one XCD; started in lockstep, all of them would wait
  // on the same first-touch misses beyond L2 in every k-step.  Each tile instead starts its k-loop
  // (m_t + n_t) % 4 k-steps in and wraps around, so neighbours sharing a row of A or W lead one
  // another by a few k-steps and mostly find the lines in L2 (prefill 23.1-23.3 -> 22.3 ms; a
  // spread over the whole K range measured 14 % slower there, the lines leaving L2 first).  The
  // order depends only on the tile, so every row's sum is the same at any batch size.
  const int koff = ((m_t + n_t) & 3) % nkt;

  // DMA sources: instruction i of this wave fills LDS rows 8*(wave*LPW + i) .. +7 of the stage;
  // lane (row r = l/8, position p = l%8) fetches chunk p ^ (r & 7) of its row
  const Op *src[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int r = (wave * LPW + i) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ (r & 7);
    const Op *row = r < BM ? A + (size_t)min(m0 + r, M - 1) * K : epi.wrow(n0 + r - BM);  // rows past M: never stored
    src[i] = row + kb + chunk * VE;
  }
  auto dma = [&](auto bufc, int kt) {
    const unsigned dst = lds_addr(big_buf<STAGE, decltype(bufc)::value>()) + wave * LPW * 1024;
#pragma unroll
    for (int i = 0; i < LPW; ++i) dma16(src[i] + ((kt + koff) % nkt) * BK, dst + i * 1024);
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment rows of this wave: A rows wm*64 + i*16 + c16, W rows BM + wn*BN/WN + j*16 + c16;
  // (row & 7) == (c16 & 7) for all of them
  const int sw = c16 & 7;
  const int arow = (wm * (BM / WM) + c16) * RB, wrow = (BM + wn * (BN / WN) + c16) * RB;

  // one k-step: wait for its loads, multiply, and start the loads NBUF-1 steps ahead into the
  // buffer read in the previous step.  With three buffers the copies go out half-way through the
  // step: issued right after the barrier, the copies of all 8 waves meet every wave's first
  // fragment reads in the LDS, issued half-way they overlap the MFMAs (a probe of this loop:
  // 58 % -> 71 % of the MFMA rate; the bf16 GEMMs 3-5 % faster).  With two buffers the copy has
  // only this one step to land, so it goes out first.
  auto step = [&](auto curc, int kt) {
    constexpr int CB = decltype(curc)::value;
    const char *cur = big_buf<STAGE, CB>();
    // the copies of the steps after kt (at most NBUF-2 of them) may stay in flight
    const int after = min(NBUF - 2, nkt - 1 - kt);
    if (NBUF >= 4 && after >= 2) vm_wait<(NBUF >= 4 ? 2 * LPW : 0)>();
    else if (NBUF >= 3 && after >= 1) vm_wait<(NBUF >= 3 ? LPW : 0)>();
    else vm_wait<0>();
    wg_barrier();  // every wave's step kt has landed; step kt-1 is fully read
    auto issue = [&] {
      if (kt + NBUF - 1 < nkt) dma(std::integral_constant<int, (CB + NBUF - 1) % NBUF>{}, kt + NBUF - 1);
    };
    if constexpr (EB == 2) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        if (kc == (NBUF >= 3 ? 1 : 0)) issue();
        const int pos = ((kc * 4 + g) ^ sw) * 16;
        bf16x8 fa[TM], fb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[i] = *reinterpret_cast<const bf16x8 *>(cur + arow + i * 16 * RB + pos);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[j] = *reinterpret_cast<const bf16x8 *>(cur + wrow + j * 16 * RB + pos);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = Mfma<bf16>::mma(fa[i], fb[j], acc[i][j]);
      }
    } else {
      issue();  // FP8: one MFMA k-chunk per step; measured slower half-way
      const int p0 = ((2 * g) ^ sw) * 16, p1 = ((2 * g + 1) ^ sw) * 16;
      i32x8 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const i32x4 lo = *reinterpret_cast<const i32x4 *>(cur + arow + i * 16 * RB + p0);
        const i32x4 hi = *reinterpret_cast<const i32x4 *>(cur + arow + i * 16 * RB + p1);
        fa[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const i32x4 lo = *reinterpret_cast<const i32x4 *>(cur + wrow + j * 16 * RB + p0);
        const i32x4 hi = *reinterpret_cast<const i32x4 *>(cur + wrow + j * 16 * RB + p1);
        fb[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = Mfma8::mma(fa[i], fb[j], acc[i][j]);
    }
  };

  static_for<0, NBUF - 1>([&](auto I) {
    if (I < nkt) dma(I, I);
  });
  epi.prepare(m0, BM, rinv);  // its loads queue behind the first stages
  int kt = 0;
  for (; kt + NBUF <= nkt; kt += NBUF) static_for<0, NBUF>([&](auto I) { step(I, kt + I); });
  static_for<0, NBUF - 1>([&](auto I) {
    if (kt + I < nkt) step(I, kt + I);
  });
  __syncthreads();  // rinv (written by epi.prepare) visible; every stage read is done

  if (sk.k_split > 1) {  // partial sums [split][M][N], row-major; resid_reduce_kernel finishes
    const int N = n_tiles * BN;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + wm * (BM / WM) + i * 16 + 4 * g + r;
          if (row < M) sk.part[((size_t)split * M + row) * N + n0 + wn * (BN / WN) + j * 16 + c16] = acc[i][j][r];
        }
    return;
  }
  if constexpr (Epi::kTile && EB == 2) {
    if (epi.tile_ok(BN)) {  // uniform
      // stage the finished tile in LDS (the k-step buffers are free now), then store whole rows;
      // up to 128 rows per pass (a 256-row tile takes two, each staged by the waves that own its
      // rows; a 64-row tile one pass of 64)
      constexpr int LD = BN + 8, PR = BM < 128 ? BM : 128;
      static_assert(64 * LD * 2 <= STAGE, "half a pass fits in one stage buffer");
      static_assert(BM % PR == 0 && (BM / WM) <= PR, "a wave's rows lie in one pass");
      const TileRows<bf16, LD> ot{reinterpret_cast<bf16 *>(big_buf<STAGE, 0>()), reinterpret_cast<bf16 *>(big_buf<STAGE, 1>())};
      static_for<0, BM / PR>([&](auto P) {
        constexpr int pass = decltype(P)::value;
        const int pm0 = m0 + pass * PR;
        if constexpr (pass > 0) __syncthreads();  // the previous pass's rows are stored
        if (wm * (BM / WM) / PR == pass) {  // uniform per wave
          // the epilogue's loads of row tile i+1 go out before row tile i is processed, so only
          // the first ones are waited for
          typename Epi::St st[2][TN];
          auto load_row_tile = [&](int i, typename Epi::St(&dst)[TN]) {
            const RowInfo ri = row_info(epi.rows(), m0 + wm * (BM / WM) + i * 16 + 4 * g, M);
#pragma unroll
            for (int j = 0; j < TN; ++j) dst[j] = epi.load(ri, n0 + wn * (BN / WN) + j * 16 + c16);
          };
          load_row_tile(0, st[0]);
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            if (i + 1 < TM) load_row_tile(i + 1, st[(i + 1) & 1]);
            const int row0 = m0 + wm * (BM / WM) + i * 16 + 4 * g;
#pragma unroll
            for (int j = 0; j < TN; j += 2)
              epi.to_lds2(st[i & 1][j], st[i & 1][j + 1], row0, n0 + wn * (BN / WN) + j * 16 + c16, acc[i][j],
                          acc[i][j + 1], rinv + pass * PR, pm0, n0, ot);
          }
        }
        __syncthreads();
        epi.template lds_out<PR, BN>(ot, pm0, n0, M);
      });
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int row0 = m0 + wm * (BM / WM) + i * 16 + 4 * g;
    if (row0 - 4 * g >= M) break;  // uniform over the wave: the whole 16-row tile is past M
    const RowInfo ri = row_info(epi.rows(), row0, M);
    typename Epi::St st[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) st[j] = epi.load(ri, n0 + wn * (BN / WN) + j * 16 + c16);
#pragma unroll
    for (int j = 0; j < TN; j += 2)
      epi.store2(st[j], st[j + 1], ri, row0, n0 + wn * (BN / WN) + j * 16 + c16, acc[i][j], acc[i][j + 1], true, rinv, m0);
  }
}

// Tiles of 128 rows x nt = 128 or 256 columns with three k-step buffers, or 384 with two (LDS
// holds only two stages of 512 rows); bf16 also 256 x 256 with two (8 waves as 4 x 2, each
// 64 x 128: a third fewer copied bytes and LDS fragment reads per MFMA than 128 x 384).
template <typename Op, class Epi>
static void run_big(const Op *A, int M, int N, int K, const Epi &epi, int nt, int bm, const SplitK &sk, hipStream_t s) {
  // 8 waves (two per SIMD: while one waits on LDS or the barrier, the other multiplies).
  // Measured: 4 waves (2 x 2) 13-14 % slower at the batch-32 shapes; 16 waves (4 x 4, 128
  // registers per lane) no faster there and the FP8 prefill 1.8 x slower.
  constexpr int NW = 8, WM = 2;
  const int nN = N / nt;
  // tile order: the band height whose run of workgroups resident on one XCD at a time (one per
  // CU, 32 per XCD) touches the fewest distinct operand rows, so more of them meet in that
  // XCD's L2 (prefill down 193 -> 167 us with bands of one row tile)
  auto group_m = [&](int bm_, int nM) {
    const long T = (long)nN * nM * sk.k_split, W = std::min<long>((T + 7) / 8, 32);
    int best = nM;
    long best_rows = -1;
    for (int g = nM; g >= 1; --g) {
      const long rows = std::min<long>(W, g) * bm_ + (W + g - 1) / g * nt;
      if (best_rows < 0 || rows < best_rows) best = g, best_rows = rows;
    }
    return best;
  };
  if constexpr (sizeof(Op) == 2 && std::is_same<Epi, EpiResid<Op>>::value) {
    // residual projections only (a 64-column tile would split the RoPE pairs of a QKV head)
    if (nt == 64) {  // 128 x 64, 8 waves as 4 x 2 (32 x 32 each), four 24 KB stages
      const int nM = (M + 127) / 128;
      dim3 grid(nN, nM, sk.k_split);
      hipLaunchKernelGGL((big_kernel<Op, 64, 4, NW, 4, 128, Epi>), grid, dim3(NW * 64), 0, s, A, M, K, epi, sk, nN, nM,
                         group_m(128, nM));
      return;
    }
  }
  if constexpr (sizeof(Op) == 2) {
    if (bm == 64) {  // 64-row tiles for a few hundred rows: twice the workgroups of 128-row ones
      const int nM = (M + 63) / 64;
      dim3 grid(nN, nM, sk.k_split);
      const int gm = group_m(64, nM);
      if (nt == 256)  // 40 KB stages, three buffers
        hipLaunchKernelGGL((big_kernel<Op, 256, 3, NW, WM, 64, Epi>), grid, dim3(NW * 64), 0, s, A, M, K, epi, sk, nN, nM, gm);
      else  // 24 KB stages, four buffers
        hipLaunchKernelGGL((big_kernel<Op, 128, 4, NW, WM, 64, Epi>), grid, dim3(NW * 64), 0, s, A, M, K, epi, sk, nN, nM, gm);
      return;
    }
  }
  if constexpr (sizeof(Op) == 2 || Epi::kTile) {  // FP8 residual tiles of 256 rows spill: not built
    if (bm == 256 && nt == 256) {
      const int nM = (M + 255) / 256;
      dim3 grid(nN, nM, sk.k_split);
      hipLaunchKernelGGL((big_kernel<Op, 256, 2, NW, 4, 256, Epi>), grid, dim3(NW * 64), 0, s, A, M, K, epi, sk, nN, nM,
                         group_m(256, nM));
      return;
    }
  }
  const int nM = (M + 127) / 128;
  dim3 grid(nN, nM, sk.k_split);
  const int gm = group_m(128, nM);
  if (nt == 384)
    hipLaunchKernelGGL((big_kernel<Op, 384, 2, NW, WM, 128, Epi>), grid, dim3(NW * 64), 0, s, A, M, K, epi, sk, nN, nM, gm);
  else if (nt == 256)
    hipLaunchKernelGGL((big_kernel<Op, 256, 3, NW, WM, 128, Epi>), grid, dim3(NW * 64), 0, s, A, M, K, epi, sk, nN, nM, gm);
  else
    hipLaunchKernelGGL((big_kernel<Op, 128, 3, NW, WM, 128, Epi>), grid, dim3(NW * 64), 0, s, A, M, K, epi, sk, nN, nM, gm);
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
    for (int j = 0; j < TN; j += 2)
      epi.store2(st[i][j], st[i][j + 1], ri[i], m0 + wm * (BM / 2) + i * 16 + 4 * (lane >> 4),
                 n0 + wn * (BN / 2) + j * 16 + (lane & 15), acc[i][j], acc[i][j + 1], true, rinv, m0);
}

template <typename T, int NT, int RT, int NWV, class Epi>
static void run_skinny_rt(const T *A, int M, int N, int K, const Epi &epi, const GemmPlan &p, hipStream_t s) {
  dim3 grid(N / NT, p.sk.k_split, (M + 16 * RT - 1) / (16 * RT));
  const int nk = K / p.sk.k_split / NWV / (4 * Mfma<T>::EPL);
  switch (nk) {
#define DM_NK(n) \
  case n: hipLaunchKernelGGL((skinny_kernel<T, NT, n, RT, NWV, Epi>), grid, dim3(NWV * 64), 0, s, A, M, K, epi, p.sk); break;
    DM_NK(1) DM_NK(2) DM_NK(3) DM_NK(4) DM_NK(5) DM_NK(6) DM_NK(7) DM_NK(8)
#undef DM_NK
    default: break;  // the host plan never asks for more than 8 k-chunks per wave
  }
}
template <typename T, int NT, class Epi>
static void run_skinny(const T *A, int M, int N, int K, const Epi &epi, const GemmPlan &p, hipStream_t s) {
  if constexpr (NT == 16 && std::is_same<Epi, EpiResid<T>>::value) {
    if (p.nw == 16) {  // residual projections whole-K per workgroup
      if (p.rt == 1) run_skinny_rt<T, NT, 1, 16>(A, M, N, K, epi, p, s);
      else run_skinny_rt<T, NT, 2, 16>(A, M, N, K, epi, p, s);
      return;
    }
  }
  if (p.rt == 2) run_skinny_rt<T, NT, 2, 4>(A, M, N, K, epi, p, s);
  else run_skinny_rt<T, NT, 4, 4>(A, M, N, K, epi, p, s);
}

template <typename T, class Epi>
static void run_gemm(const T *A, int M, int N, int K, const Epi &epi, const GemmPlan &p, hipStream_t s) {
  if (p.skinny) {
    switch (p.nt) {
      case 16: run_skinny<T, 16>(A, M, N, K, epi, p, s); break;
      case 32: run_skinny<T, 32>(A, M, N, K, epi, p, s); break;
      default: run_skinny<T, 64>(A, M, N, K, epi, p, s); break;
    }
  } else if (p.nt >= 64) {
    if constexpr (std::is_same<T, bf16>::value) {
      run_big<bf16>(A, M, N, K, epi, p.nt, p.bm, p.sk, s);
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
    const dim3 grid((n + 255) / 256);
    switch (p.sk.k_split) {
      case 2: hipLaunchKernelGGL((resid_reduce_kernel<T, 2>), grid, dim3(256), 0, s, a, p.sk.part); break;
      case 4: hipLaunchKernelGGL((resid_reduce_kernel<T, 4>), grid, dim3(256), 0, s, a, p.sk.part); break;
      case 8: hipLaunchKernelGGL((resid_reduce_kernel<T, 8>), grid, dim3(256), 0, s, a, p.sk.part); break;
      default: hipLaunchKernelGGL((resid_reduce_kernel<T, 16>), grid, dim3(256), 0, s, a, p.sk.part); break;
    }
  }
}
template <typename T> static void swiglu_t(const SwigluArgs &a, const GemmPlan &p, hipStream_t s) {
  run_gemm<T>((const T *)a.in.hg, a.M, 2 * a.F, a.in.H, EpiSwiglu<T>{a}, p, s);
}

// FP8: one launch of the large-tile kernel, 256 columns per workgroup when N allows it.
template <class Epi> static void run_fp8(const fp8 *A, int M, int N, int K, const Epi &epi, hipStream_t s) {
  const SplitK none{1, nullptr};
  const int nt = N % 256 == 0 ? 256 : 128;
  // gate/up: 256 x 256 while those still make ~200 workgroups (an FP8 k-step's MFMAs take half
  // the time of bf16's for the same copied bytes, so reuse per byte matters twice as much; the
  // prefill's gate/up 266 -> 220 us).  The residual epilogue keeps 128 rows (256 rows spill
  // registers and measured 4 % slower).
  const int bm = Epi::kTile && nt == 256 && (size_t)(N / 256) * ((M + 255) / 256) >= 200 ? 256 : 128;
  run_big<fp8>(A, M, N, K, epi, nt, bm, none, s);
}
void launch_resid_fp8(const ResidArgs &a, hipStream_t s) {
  run_fp8((const fp8 *)a.a, a.M, a.out.H, a.K, EpiResid<bf16, fp8>{a}, s);
}
void launch_swiglu_fp8(const SwigluArgs &a, hipStream_t s) {
  run_fp8((const fp8 *)a.a8, a.M, 2 * a.F, a.in.H, EpiSwiglu<bf16, fp8>{a}, s);
}

int gemm_k_quantum(Dt dt) { return 4 * 4 * (dt == DT_BF16 ? Mfma<bf16>::EPL : Mfma<float>::EPL); }

// Qwen3 per-head QK-norm, then rotate-half RoPE, in place on the Q and K the product wrote
// unrotated: workgroup = (row, head), lane i < D/2 the pair (i, i + D/2); rows past a sample's
// prefix are left untouched, as by the product.
template <typename T> __global__ __launch_bounds__(64) void qk_norm_rope_kernel(QkvArgs a) {
  const int m = blockIdx.x, h = blockIdx.y, i = threadIdx.x, half = a.D >> 1;
  const int rpb = a.rows.rows_per_b, b = m / rpb, s = m - b * rpb;
  if (a.rows.is_prefix && s >= max(0, min(a.rows.lens[b], a.rows.cap))) return;  // uniform
  T *p;
  const float *g;
  if (h < a.Hq) {
    p = (T *)a.q + (size_t)m * a.Hq * a.D + (size_t)h * a.D;
    g = a.q_norm;
  } else {
    p = (T *)a.k + ((size_t)(b * a.Hkv + h - a.Hq) * a.kv_rows + s) * a.D;
    g = a.k_norm;
  }
  const bool on = i < half;
  const float x0 = on ? to_f32(p[i]) : 0.f, x1 = on ? to_f32(p[i + half]) : 0.f;
  const float inv = rsqrtf(wave_sum(x0 * x0 + x1 * x1) / (float)a.D + a.eps);
  if (!on) return;
  const float n0 = x0 * inv * g[i], n1 = x1 * inv * g[i + half];
  const float2 cs = a.rows.is_prefix ? a.rope[(size_t)s * half + i] : a.rope_rows[(size_t)m * half + i];
  p[i] = from_f32<T>(n0 * cs.x - n1 * cs.y);
  p[i + half] = from_f32<T>(n1 * cs.x + n0 * cs.y);
}

void launch_qkv(Dt dt, const QkvArgs &a, const GemmPlan &p, hipStream_t s) {
  if (dt == DT_BF16) qkv_t<bf16>(a, p, s); else qkv_t<float>(a, p, s);
  if (a.q_norm) {
    const dim3 grid(a.M, a.Hq + a.Hkv);
    if (dt == DT_BF16) hipLaunchKernelGGL(qk_norm_rope_kernel<bf16>, grid, dim3(64), 0, s, a);
    else hipLaunchKernelGGL(qk_norm_rope_kernel<float>, grid, dim3(64), 0, s, a);
  }
}
void launch_resid(Dt dt, const ResidArgs &a, const GemmPlan &p, hipStream_t s) {
  if (dt == DT_BF16) resid_t<bf16>(a, p, s); else resid_t<float>(a, p, s);
}
void launch_swiglu(Dt dt, const SwigluArgs &a, const GemmPlan &p, hipStream_t s) {
  if (dt == DT_BF16) swiglu_t<bf16>(a, p, s); else swiglu_t<float>(a, p, s);
}

}  // namespace dm

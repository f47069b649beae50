// Batch-1 suffix denoise of the DM0-base action expert in ONE kernel launch per action chunk.
//
// Pages: "DM0 paper definition vs. Dexbotic code", section 1 (each expert's own Q/K/V, joint
// attention over [prefix ; action] keys, own O-projection, residual and MLP; 28 layers, hidden
// 1024, 16 query heads over 8 KV heads of dim 128); "DM0.5: High-Performance Embodied VLA and
// OpenDM Open Source Introduction", sections 5.1-5.3 (the cached prefix K/V, action_in_proj /
// action_out_proj, Euler integration over diffusion_steps) and 6.4 (at small batch the cost lies
// in the many per-step launches and temporaries, not in arithmetic).
//
// At one sample a layer-step moves about 34 MB (weights and the prefix K/V) but does only
// ~60 MFLOP, and its five products depend on each other, so separate kernels spend most of their
// time starting up, refilling caches and waiting on the previous launch.  Here 256 workgroups (one
// per CU, all resident) run the whole chunk: 10 Euler steps x 28 layers.  Each workgroup owns a
// fixed slice of every weight matrix and of the prefix K/V (persist_plan.h), and four of its
// waves do nothing but copy those slices from HBM into LDS one layer ahead (global_load_lds), so
// the weight stream runs while the other eight waves wait on their inputs.
//
// The workgroups form 8 groups of 32 (group x = block % 8 = the XCD it runs on).  Group x works
// like one rank of a tensor-parallel layer: it owns KV head x (query heads 2x and 2x+1), FFN
// columns 384x..384x+383 and a full copy of the residual stream.  A layer is eight phases:
//   P1 QKV      Q/K/V of head x for all action tokens (RMSNorm row scale, RoPE)   group barrier
//   P2 attention key chunk i of head x over all 2 x S query slots               group barrier
//   P3 merge    the 32 chunk partials of head x (log-sum-exp weights)            group barrier
//   P4 O-part   O-projection of head x's 256 inputs -> a partial of all 1024 cols  (tagged data)
//   P5 reduce   workgroup i: h[:, 32i..] += sum of the 8 groups' partials, h*gain  group barrier
//   P6 gate/up  SwiGLU of FFN columns 384x + 12i .. +11                          group barrier
//   P7 D-part   down-projection of group x's 384 FFN inputs -> partial of all cols  (tagged data)
//   P8 reduce   as P5 (then the next layer's norm gain)                          group barrier
// and each Euler step adds the velocity head (its partial in P8 of the last layer, a reduce +
// Euler update, then action_in_proj + time embedding of the next step).  Only P4->P5 and P7->P8
// cross groups: there a workgroup reads the columns it owns from the 8 workgroups (x', i) that
// wrote them, and polls those values themselves: every fp32 partial carries the layer-step's
// epoch in its two low mantissa bits, so no separate signal (and no wait for the writes to
// complete before it) is needed.
//
// Memory model: every value one workgroup hands to another is loaded with device-coherent (sc1)
// buffer loads and stored device-coherent or, inside a group placed on one XCD, plainly into that
// XCD's L2 (no L2 write-back or invalidate is issued); before a group barrier a producer's stores
// are complete (s_waitcnt vmcnt(0)); a tagged partial needs no ordering at all, since each
// 4-byte word is checked on its own.  Weights and the prefix
// K/V are read-only and use ordinary cached copies.  Every wait is bounded: a workgroup that
// waits longer than its limit (e.g. the 256 workgroups were not all resident) records an error,
// every workgroup leaves, and the chunk is filled with NaN.  Reductions run in a fixed order, so
// results are bitwise reproducible.
#include <cmath>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "persist_plan.h"

namespace dm {
namespace pk {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((ext_vector_type(2))) int i32x2;
constexpr int SC1 = 16;  // cache-policy bits of a device-coherent buffer access

// LDS map (bytes)
constexpr int L_QKV = 0;
constexpr int L_KV = L_QKV + SEG_BYTES[SEG_QKV];
constexpr int L_O = L_KV + SEG_BYTES[SEG_KV];
constexpr int L_GU = L_O + SEG_BYTES[SEG_O];
constexpr int L_D = L_GU + SEG_BYTES[SEG_GU];
constexpr int L_RED = L_D + SEG_BYTES[SEG_D];   // cross-wave partial sums: 2 tiles x 4 waves x 1 KB
constexpr int L_ROPE = L_RED + 8192;             // (cos, sin) [SMAX tokens][8 pairs]
constexpr int L_INV = L_ROPE + SMAX * 8 * 8;     // 1/rms per token
constexpr int L_FLAG = L_INV + SMAX * 4;         // abort flag
constexpr int L_GAIN = L_FLAG + 64;              // norm gains of this workgroup's 32 columns:
                                                 // [LMAX][2][32] (attention, MLP), then final norm
constexpr int L_TOTAL = L_GAIN + (LMAX * 2 + 1) * HC * 4;
static_assert(L_TOTAL <= 160 * 1024, "LDS budget");
constexpr int SEG_LDS[NSEG] = {L_QKV, L_KV, L_O, L_GU, L_D};

constexpr long MAX_POLLS = 1L << 21;     // ~2 s of polling: far beyond any legitimate wait
constexpr int OUT_OF_RANGE = 0x40000000;  // a buffer offset past every workspace

__device__ __forceinline__ rsrc_t mkrsrc(const void *p, long bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ i32x4 ld16(rsrc_t r, int off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, SC1); }
__device__ __forceinline__ i32x2 ld8(rsrc_t r, int off) { return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, SC1); }
__device__ __forceinline__ float ld4f(rsrc_t r, int off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, SC1));
}
__device__ __forceinline__ void st16(rsrc_t r, int off, i32x4 v) { __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, SC1); }
__device__ __forceinline__ void st8(rsrc_t r, int off, i32x2 v) { __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, SC1); }
__device__ __forceinline__ void st4f(rsrc_t r, int off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), r, off, 0, SC1);
}
// Stores of values only workgroups of the same group read: with the group on one XCD (checked at
// start-up) a plain store lands in the XCD's shared L2, where the readers' device-coherent loads
// find it; otherwise the store is device-coherent too.
__device__ __forceinline__ void stl16(bool l2, rsrc_t r, int off, i32x4 v) {
  if (l2) __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
  else __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, SC1);
}
__device__ __forceinline__ void stl8(bool l2, rsrc_t r, int off, i32x2 v) {
  if (l2) __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
  else __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, SC1);
}
__device__ __forceinline__ void stl4f(bool l2, rsrc_t r, int off, float v) {
  if (l2) __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), r, off, 0, 0);
  else __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), r, off, 0, SC1);
}
// dma16 (global -> LDS, 16 bytes per lane) with the non-temporal hint: each weight and cached
// key is read once per layer-step, so its lines are streamed rather than kept in L2 ahead of the
// hand-off buffers.
__device__ __forceinline__ void dma16_stream(const void *g, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
template <int N> using Lines = std::integral_constant<int, N>;
template <int N> using Ph = std::integral_constant<int, N>;
__device__ __forceinline__ unsigned xcc_id() {
  unsigned v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v;
}
__device__ __forceinline__ int ld_flag(int *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_flag(int *p, int v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

__device__ __forceinline__ bf16x8 as_bf16x8(i32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ i32x2 pack4(float a, float b, float c, float d) {
  bf16x4 o;
  o[0] = (bf16)a; o[1] = (bf16)b; o[2] = (bf16)c; o[3] = (bf16)d;
  return __builtin_bit_cast(i32x2, o);
}
__device__ __forceinline__ float bf_to_f(bf16 v) { return to_f32(v); }

// sum / max over aligned groups of 8 lanes
__device__ __forceinline__ float sum8(float v) {
  v = sum4(v);
  return v + dpp<DPP_HALF_MIRROR>(v);
}
__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, dpp<DPP_XOR1>(v));
  v = fmaxf(v, dpp<DPP_XOR2>(v));
  return fmaxf(v, dpp<DPP_HALF_MIRROR>(v));
}

// value of lane l ^ 32: v_permlane32_swap of the register with itself returns the lane's own
// value and its partner's, one in each result; whichever is not bitwise the own value is the
// partner's (if both are equal, either is)
__device__ __forceinline__ float xor32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0] == __float_as_uint(v) ? p[1] : p[0]);
}

// Transposing LDS read (gfx950): per group of 16 lanes, lane i receives element i % 4 of the
// 8-byte row addressed by lane 4e + i / 4 of its group (e = 0..3).
typedef short s4v __attribute__((ext_vector_type(4)));
typedef short s8v __attribute__((ext_vector_type(8)));
__device__ __forceinline__ s4v lds_tr16(const char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4v *)p);
}

}  // namespace pk

struct PkArgs {
  const bf16 *w_qkv, *w_o, *w_gate, *w_up, *w_down;  // stacked layers, [out][in]
  const float *attn_norm, *mlp_norm;                 // [L][H]
  const float *w_in, *b_in, *final_norm, *w_out, *b_out;
  const bf16 *k_cache, *v_cache;                     // [L][1][Hkv][P_cap][D]
  const int32_t *lens;                               // [1]
  float *x;                                          // [S][A]
  int L, S, A, P_cap, steps;
  float eps, rope_base;
  // workspace regions (device-coherent hand-offs): byte offsets from ws_base
  char *ws_base; int ws_bytes;
  int off_hg, off_ssq, off_qkv, off_apart, off_aml, off_o, off_opart, off_act, off_dpart, off_vpart, off_xs;
  int *sync;
};

namespace pk {

// sync area (ints): [0, 8*64): group counters (one 256-byte line each); then the error word, the
// start-up arrival counter and the placement word, each on its own 256-byte line
constexpr int SYNC_CNT = 0, SYNC_ERR = 512, SYNC_START = SYNC_ERR + 64, SYNC_MISPLACED = SYNC_START + 64,
              SYNC_INTS = SYNC_MISPLACED + 64;

// Waits (one lane) until every int at p[k * stride], k < n, is >= target; bounded.  Returns
// false on timeout or when another workgroup has recorded an error.
__device__ __forceinline__ bool wait_geq(int *p, int stride, int n, int target, int *err) {
  long polls = 0;
  while (true) {
    bool ok = true;
    for (int k = 0; k < n; ++k) ok &= ld_flag(p + k * stride) >= target;
    if (ok) return true;
    if ((++polls & 31) == 0 && ld_flag(err) != 0) return false;
    if (polls >= MAX_POLLS) {
      st_flag(err, 1);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// The body, instantiated once for the compute waves (CW) and once for the copy waves: both run
// the same sequence of phases and workgroup barriers (the same code, each role's work pruned at
// compile time), so their barriers pair up while their registers are allocated separately.
// An opaque copy of v: values derived from it are recomputed where they are used instead of
// being hoisted out of the layer loop and kept live across every phase.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

template <bool CW>
__device__ __forceinline__ void pk_run(const PkArgs &a, char *smem) {
  const int tid = threadIdx.x;
  int lane = tid & 63, wave = tid >> 6;
  int g = lane >> 4, c16 = lane & 15;
  constexpr bool cw = CW;              // compute wave
  const int dw = wave - NCW;           // copy wave index (0..3) when !cw
  const int b = blockIdx.x, x = b & (NX - 1), i = b >> 3;
  const int S = a.S, A = a.A, L = a.L, N = a.steps;
  const int P = max(0, min(a.lens[0], a.P_cap));
  const int Pc = prefix_chunk(P), Sc = action_chunk(S);
  int tt = wave & 3, hw = (wave >> 2) & 1;  // compute waves: token tile, K half / row tile
  // residual slice of thread tid < 8*S: token ht, columns hc .. hc+3 (see the residual slice below)
  int ht = tid >> 3, hc = HC * i + 4 * (tid & 7);
  bool l2 = false;  // intra-group hand-offs through L2 (set at start-up)
  int *sync = a.sync;
  int *err = sync + SYNC_ERR;
  int *cnt = sync + SYNC_CNT + 64 * x;
  int *abort_lds = reinterpret_cast<int *>(smem + L_FLAG);
  float *inv = reinterpret_cast<float *>(smem + L_INV);

  // device-coherent view of the hand-off buffers: one buffer resource over the workspace, each
  // region a byte offset (a buffer access past the workspace reads 0 and writes nothing)
  const rsrc_t rw = mkrsrc(a.ws_base, a.ws_bytes);
  const int o_hg = a.off_hg + x * S * H * 2, o_ssq = a.off_ssq + x * S * (H / 16) * 4;
  const int o_qkv = a.off_qkv + x * S * GW * 2, o_ap = a.off_apart + x * NG * 2 * S * D * 2;
  const int o_am = a.off_aml + x * NG * 2 * S * 8, o_o = a.off_o + x * S * 2 * D * 2;
  const int o_opart = a.off_opart, o_act = a.off_act + x * S * FG * 2, o_dpart = a.off_dpart;
  const int o_vp = a.off_vpart + x * NG * S * A * 4, o_xs = a.off_xs + x * S * A * 4;

  // ------------------------------------------------------------------ copy (DMA) waves
  // Lines [u0, u1) of this copy wave's share of segment `seg` (1 KB each) for layer-step ls.
  auto issue = [&](auto segc, int ls, auto u0c, auto u1c) {
    constexpr int seg = decltype(segc)::value;
    const int l = ls % L;
    constexpr int per = SEG_LINES[seg] / NDW;
    constexpr int u0 = decltype(u0c)::value, u1 = decltype(u1c)::value;
    static_assert(0 <= u0 && u0 < u1 && u1 <= per, "line range");
    const unsigned base = lds_addr(smem + SEG_LDS[seg]);
#pragma unroll
    for (int u = u0; u < u1; ++u) {
      const int line = dw * per + u;
      const char *src;
      if constexpr (seg == SEG_KV) {
        int is_v;
        const long e = kv_piece(i, Pc, P, line, lane, &is_v);
        const bf16 *blk = (is_v ? a.v_cache : a.k_cache) + ((long)l * HKV + x) * a.P_cap * D;
        src = (const char *)(blk + e);
      } else {
        int which;
        const long e = weight_piece(seg, x, i, line, lane, &which);
        const bf16 *w;
        if constexpr (seg == SEG_QKV) w = a.w_qkv + (long)l * QKV_ROWS * H;
        else if constexpr (seg == SEG_O) w = a.w_o + (long)l * H * HQ * D;
        else if constexpr (seg == SEG_GU) w = (which ? a.w_up : a.w_gate) + (long)l * F * H;
        else w = a.w_down + (long)l * H * F;
        src = (const char *)(w + e);
      }
      dma16_stream(src, base + line * 1024);
    }
  };
  const int total_ls = N * L;
  // What a copy wave does at the start of phase PH of layer-step ls: the pieces and the wait of
  // COPY_PLAN / COPY_WAIT (persist_plan.h, where the schedule is explained).
  auto copy_step = [&](auto phc, int ls) {
    constexpr int ph = decltype(phc)::value;
    if constexpr (cw || ph >= NPH) {
      return;
    } else {
      const bool more = ls + 1 < total_ls;
      auto piece = [&](auto kc) {
        constexpr CopyPiece c = COPY_PLAN[ph][decltype(kc)::value];
        if constexpr (c.seg >= 0) {
          if (c.next == 0 || more)
            issue(std::integral_constant<int, c.seg>{}, ls + c.next, Lines<c.u0>{}, Lines<c.u1>{});
        }
      };
      piece(std::integral_constant<int, 0>{});
      piece(std::integral_constant<int, 1>{});
      if constexpr (COPY_WAIT[ph] >= 0) {
        if (more) vm_wait<COPY_WAIT[ph]>();
        else vm_wait<0>();
      }
    }
  };
  static_assert(COPY_PIECES == 2, "copy_step issues two pieces per phase");
  using QKVs = std::integral_constant<int, SEG_QKV>;
  using KVs = std::integral_constant<int, SEG_KV>;
  using Os = std::integral_constant<int, SEG_O>;
  using GUs = std::integral_constant<int, SEG_GU>;
  using Ds = std::integral_constant<int, SEG_D>;

  // ------------------------------------------------------------------ synchronisation
  int n_bar = 0;  // group barriers passed
  // Phase entry: lane 0 of wave 0 waits for the group barrier (group phases) or only checks the
  // error word (the two reduces, which poll their tagged inputs themselves), the copy waves do
  // their copy step; then one workgroup barrier.  Returns false when the chunk is aborted.
  auto enter = [&](auto ph, int ls, bool group) {
    lane = opaque(tid) & 63;  // lane-derived addresses are rebuilt in every phase
    wave = opaque(tid) >> 6;
    g = lane >> 4;
    c16 = lane & 15;
    tt = wave & 3;
    hw = (wave >> 2) & 1;
    ht = opaque(tid) >> 3;
    hc = HC * i + 4 * (opaque(tid) & 7);
    if (tid == 0) {
      bool ok;
      if (group) ok = wait_geq(cnt, 0, 1, NG * n_bar, err);
      else ok = ld_flag(err) == 0;
      *abort_lds = ok ? 0 : 1;
    }
    copy_step(ph, ls);
    __syncthreads();
    return *abort_lds == 0;
  };
  // Phase exit: the compute waves' stores are complete, then lane 0 arrives at the group counter.
  auto leave_group = [&]() {
    if (cw) vm_wait<0>();
    __syncthreads();
    ++n_bar;
    if (tid == 0) __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  // Exit of a phase whose outputs are tagged partials: nothing to wait for or signal.
  auto leave_plain = [&]() { __syncthreads(); };
  // The partials' epoch: layer-step ls modulo 4 in the two low mantissa bits of every float (a
  // change of at most 3 ulp).  Every element is rewritten every layer-step by the same lane, so a
  // reader sees either the previous layer-step's tag or this one's; before the first layer-step
  // the buffers hold all-ones (tag 3).
  auto tag_bits = [](f32x4 v, int ls) {
    i32x4 u = __builtin_bit_cast(i32x4, v);
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = (u[j] & ~3) | (ls & 3);
    return u;
  };
  auto poll_tagged = [&](i32x4 *pv, int off, int ls) {
    const int tag = ls & 3;
    long polls = 0;
    while (true) {
      int bad = 0;
#pragma unroll
      for (int xx = 0; xx < NX; ++xx) {
        const bool okx = ((pv[xx][0] & 3) == tag) & ((pv[xx][1] & 3) == tag) & ((pv[xx][2] & 3) == tag) & ((pv[xx][3] & 3) == tag);
        bad |= okx ? 0 : (1 << xx);
      }
      if (!bad) return;
      if ((++polls & 31) == 0 && ld_flag(err) != 0) return;
      if (polls >= MAX_POLLS) { st_flag(err, 1); return; }
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int xx = 0; xx < NX; ++xx)
        if (bad & (1 << xx)) pv[xx] = ld16(rw, off + ((xx * S + ht) * H + hc) * 4);
    }
  };

  // ------------------------------------------------------------------ GEMM pieces
  // A fragment of weight segment rows 16*rt + c16 (LDS layout [kstep][R][128 B], swizzled) at
  // k-chunk kc (32 inputs).
  auto afrag = [&](int lds_off, int R, int row, int kc) {
    const int chunk = (kc & 1) * 4 + g;
    return *reinterpret_cast<const bf16x8 *>(smem + lds_off + ((kc >> 1) * R + row) * 128 + ((chunk ^ (row & 7)) << 4));
  };
  // B fragment: activation [S][ld] bf16 (device-coherent), token tile tt, inputs k .. k+31.  Rows
  // past S take an offset beyond the workspace: the buffer load returns 0 without a memory access.
  auto bfrag = [&](int off, int ld, int k) {
    const int tok = 16 * tt + c16;
    return as_bf16x8(ld16(rw, tok < S ? off + (tok * ld + k + 8 * g) * 2 : OUT_OF_RANGE));
  };
  // 1/rms of every token from the group's per-16-column sums of squares, into LDS: the loads
  // (issued after the phase's operand loads, so they share one round trip), then the sums
  struct Rms { i32x4 u0, u1; };
  auto rms_issue = [&]() {
    Rms r{};
    if (cw && tid < 8 * S) {
      const int t = tid >> 3, part = tid & 7;
      r.u0 = ld16(rw, o_ssq + (t * (H / 16) + part * 8) * 4);
      r.u1 = ld16(rw, o_ssq + (t * (H / 16) + part * 8 + 4) * 4);
    }
    return r;
  };
  auto rms_finish = [&](const Rms &r) {
    if (cw && tid < 8 * S) {
      const int t = tid >> 3, part = tid & 7;
      const f32x4 v0 = __builtin_bit_cast(f32x4, r.u0), v1 = __builtin_bit_cast(f32x4, r.u1);
      float s = ((v0[0] + v0[1]) + (v0[2] + v0[3])) + ((v1[0] + v1[1]) + (v1[2] + v1[3]));
      s = sum8(s);
      if (part == 0) inv[t] = rsqrtf(s / (float)H + a.eps);
    }
  };

  // ------------------------------------------------------------------ residual slice
  // Thread tid < 8*S owns h[t][32i + c4 .. +3] (t = tid / 8, c4 = 4 (tid % 8)) for the whole
  // chunk, in registers: every group keeps an identical copy of the residual stream.
  const bool hown = cw && tid < 8 * S;
  f32x4 h4 = {0.f, 0.f, 0.f, 0.f};
  // hg = bf16(h * gain), sums of squares per 16 columns (4 threads), both device-coherent
  const float *gains = reinterpret_cast<const float *>(smem + L_GAIN);
  auto gain_attn = [&](int l) { return gains + (2 * l) * HC; };
  auto gain_mlp = [&](int l) { return gains + (2 * l + 1) * HC; };
  auto publish_h = [&](const float *gain) {  // gain: LDS slice of this workgroup's 32 columns
    if (!hown) return;
    if (gain) {
      const float4 gv = *reinterpret_cast<const float4 *>(gain + (hc - HC * i));
      stl8(l2, rw, o_hg + (ht * H + hc) * 2, pack4(h4[0] * gv.x, h4[1] * gv.y, h4[2] * gv.z, h4[3] * gv.w));
    }
    const float q = sum4(h4[0] * h4[0] + h4[1] * h4[1] + h4[2] * h4[2] + h4[3] * h4[3]);
    if ((tid & 3) == 0) stl4f(l2, rw, o_ssq + (ht * (H / 16) + hc / 16) * 4, q);
  };

  // action values owned for the Euler update: x[idx] for idx = i*per2 + tid
  const int per2 = (S * A + NG - 1) / NG;
  const int xi = i * per2 + tid;
  const bool xown = cw && tid < per2 && xi < S * A;
  float xv = xown ? a.x[xi] : 0.f;

  // ------------------------------------------------------------------ start-up
  if (cw && i < 24) {  // RoPE (cos, sin) of this workgroup's 8 pairs at positions P + t
    const int p8 = i & 7;
    float2 *rope = reinterpret_cast<float2 *>(smem + L_ROPE);
    for (int e = tid; e < S * 8; e += NCW * 64) {
      const int t = e >> 3, r = e & 7, pair = 8 * p8 + r;
      const double theta = pow((double)a.rope_base, -2.0 * pair / D);
      const double ang = (double)(P + t) * theta;
      rope[e] = make_float2((float)cos(ang), (float)sin(ang));
    }
  }
  // Placement: group x's intra-group hand-offs may stay in L2 only if all 256 workgroups run on the
  // XCD their group number names.  One arrival of every workgroup settles it (bounded wait).
  int *l2_lds = abort_lds + 1;
  if (tid == 0) {
    if ((xcc_id() & (NX - 1)) != (unsigned)x) __hip_atomic_fetch_or(sync + SYNC_MISPLACED, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(sync + SYNC_START, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool ok = wait_geq(sync + SYNC_START, 0, 1, NWG, err);
    *l2_lds = ok && ld_flag(sync + SYNC_MISPLACED) == 0;
  }
  if (cw) {  // norm gains of this workgroup's columns, every layer, into LDS
    float *gt = reinterpret_cast<float *>(smem + L_GAIN);
    for (int e = tid; e < (2 * L + 1) * HC; e += NCW * 64) {
      const int row = e / HC, c = e - row * HC;
      const float *src = row == 2 * L ? a.final_norm : ((row & 1) ? a.mlp_norm : a.attn_norm) + (long)(row >> 1) * H;
      gt[(row == 2 * L ? 2 * LMAX : row) * HC + c] = src[HC * i + c];
    }
  }
  if (!cw) {  // the first layer-step's segments, in consumption order
    issue(QKVs{}, 0, Lines<0>{}, Lines<SEG_LINES[SEG_QKV] / NDW>{});
    issue(KVs{}, 0, Lines<0>{}, Lines<SEG_LINES[SEG_KV] / NDW>{});
    issue(Os{}, 0, Lines<0>{}, Lines<SEG_LINES[SEG_O] / NDW>{});
    issue(GUs{}, 0, Lines<0>{}, Lines<SEG_LINES[SEG_GU] / NDW>{});
    issue(Ds{}, 0, Lines<0>{}, Lines<SEG_LINES[SEG_D] / NDW>{});
  }

  // action_in_proj + bias + time embedding of step k (t = 1 - k/N), h*gain of layer 0
  auto embed = [&](int k, bool from_input) {
    if (!hown) return;
    const float tk = 1.0f - (float)k / (float)N;
    f32x4 xr[AMAX / 4];
#pragma unroll
    for (int q = 0; q < AMAX / 4; ++q) {
      const int qq = min(q, A / 4 - 1);  // unconditional loads (clamped) stay in flight together
      xr[q] = from_input ? __builtin_bit_cast(f32x4, *reinterpret_cast<const float4 *>(a.x + ht * A + 4 * qq))
                         : __builtin_bit_cast(f32x4, ld16(rw, o_xs + (ht * A + 4 * qq) * 4));
    }
#pragma unroll 1
    for (int e = 0; e < 4; ++e) {
      const int c = hc + e;
      const float4 *wr = reinterpret_cast<const float4 *>(a.w_in + (long)c * A);
      float acc = 0.f;
#pragma unroll
      for (int q = 0; q < AMAX / 4; ++q)
        if (4 * q < A) {
          const float4 wv = wr[q];
          acc += wv.x * xr[q][0] + wv.y * xr[q][1] + wv.z * xr[q][2] + wv.w * xr[q][3];
        }
      const int jj = c < H / 2 ? c : c - H / 2;
      const float w = exp2f(-2.0f * (float)jj / (float)H * 13.287712379549449f);  // 10000^(-2j/H)
      const float tau = c < H / 2 ? sinf(tk * w) : cosf(tk * w);
      const float hv = acc + a.b_in[c] + tau;
      h4[0] = e == 0 ? hv : h4[0];
      h4[1] = e == 1 ? hv : h4[1];
      h4[2] = e == 2 ? hv : h4[2];
      h4[3] = e == 3 ? hv : h4[3];
    }
  };

  bool alive = true;
  // ---- step 0 entry
  embed(0, true);
  __syncthreads();  // gain tables and the placement word in LDS
  l2 = *l2_lds != 0;
  publish_h(gain_attn(0));
  leave_group();

  for (int k = 0; k < N && alive; ++k) {
    for (int l = 0; l < L && alive; ++l) {
      const int ls = k * L + l;
      // ================================================================ P1: QKV
      if (!(alive = enter(Ph<PH_QKV>{}, ls, true))) break;
      {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (cw) {
          bf16x8 bf[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) bf[u] = bfrag(o_hg, H, 32 * (16 * hw + u));
          const Rms rr = rms_issue();
#pragma unroll
          for (int u = 0; u < 16; ++u) acc = Mfma<bf16>::mma(afrag(L_QKV, 16, c16, 16 * hw + u), bf[u], acc);
          if (hw == 1) *reinterpret_cast<f32x4 *>(smem + L_RED + (tt * 64 + lane) * 16) = acc;
          rms_finish(rr);
        }
        __syncthreads();
        if (cw && hw == 0) {
          acc += *reinterpret_cast<const f32x4 *>(smem + L_RED + (tt * 64 + lane) * 16);
          const int t = 16 * tt + c16;
          const float s = inv[min(t, S - 1)];
          float y[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] = acc[j] * s;
          if (i < 24) {  // rotate-half RoPE: rows r (lanes 0..31) and r + 8 (lanes 32..63) are a pair
            const float2 *rope = reinterpret_cast<const float2 *>(smem + L_ROPE);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float other = xor32(y[j]);  // the partner lane's value
              const float2 cs = rope[min(t, S - 1) * 8 + 4 * (g & 1) + j];
              y[j] = g < 2 ? y[j] * cs.x - other * cs.y : y[j] * cs.x + other * cs.y;
            }
          }
          if (t < S) stl8(l2, rw, o_qkv + (t * GW + qkv_local_col(i, 4 * g)) * 2, pack4(y[0], y[1], y[2], y[3]));
        }
      }
      leave_group();

      // ================================================================ P2: attention chunk i
      if (!(alive = enter(Ph<PH_ATT>{}, ls, true))) break;
      {
        const int nkp = max(0, min(Pc, P - i * Pc));  // prefix keys of this chunk
        const int s0 = i * Sc, nks = max(0, min(Sc, S - s0));
        const int nk = nkp + nks;
        char *Kb = smem + L_KV, *Vb = smem + L_KV + KROWS * 256;
        // value rows past the chunk's keys are zeroed: their probabilities are 0, but a copied row
        // that is not a key (an empty prefix) may hold anything, and 0 * NaN is NaN
        if (cw && tid < (KROWS - nk) * 16) {
          const int r = nk + (tid >> 4), c = tid & 15;
          *reinterpret_cast<i32x4 *>(Vb + r * 256 + ((c ^ kv_swz(r)) << 4)) = i32x4{0, 0, 0, 0};
        }
        if (wave == NCW - 1 && lane < 2 * SC_MAX * 16) {  // action keys -> LDS rows nkp ..
          const int j = lane >> 5, isv = (lane >> 4) & 1, c = lane & 15;
          if (j < nks) {
            const i32x4 v = ld16(rw, o_qkv + ((s0 + j) * GW + (isv ? 3 : 2) * D + c * 8) * 2);
            const int r = nkp + j;
            *reinterpret_cast<i32x4 *>((isv ? Vb : Kb) + r * 256 + ((c ^ kv_swz(r)) << 4)) = v;
          }
        }
        // queries: slot = 16 w + c16 < 2S (slot / S = query head within the group, slot % S = row)
        const int slot = 16 * wave + c16;
        const bool att = cw && 16 * wave < 2 * S;
        bf16x8 qf[4];
        if (att) {
          const int sl = min(slot, 2 * S - 1), qh = sl / S, row = sl - qh * S;
#pragma unroll
          for (int dc = 0; dc < 4; ++dc) qf[dc] = as_bf16x8(ld16(rw, o_qkv + (row * GW + qh * D + 32 * dc + 8 * g) * 2));
        }
        __syncthreads();  // action keys in LDS
        if (att) {
          f32x4 st[2];
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const int kr = (c16 >> 2) * 8 + (c16 & 3) + 4 * s;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dc = 0; dc < 4; ++dc) {
              const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(Kb + kr * 256 + (((dc * 4 + g) ^ kv_swz(kr)) << 4));
              acc = Mfma<bf16>::mma(kf, qf[dc], acc);
            }
            st[s] = acc;
          }
          // lane group g holds keys 8g + 4s + j of its slot column
          const float sc = 1.4426950408889634f / sqrtf((float)D);
          float mx = -INFINITY;
#pragma unroll
          for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              if (8 * g + 4 * s + j >= nk) st[s][j] = -INFINITY;
              mx = fmaxf(mx, st[s][j]);
            }
          mx = max_xor32(max_xor16(mx)) * sc;
          const float mu = mx == -INFINITY ? 0.f : mx;
          float lsum = 0.f;
          bf16x8 pf;
#pragma unroll
          for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float p = __builtin_amdgcn_exp2f(fmaf(st[s][j], sc, -mu));
              lsum += p;
              pf[4 * s + j] = (bf16)p;
            }
          lsum = sum_xor32(sum_xor16(lsum));
          // O^T = V^T P^T over the 32 key rows
          const int vr = g * 8 + (c16 >> 2);
          const int vsw0 = kv_swz(vr), vsw1 = kv_swz(vr + 4);
          const int vpiece = (c16 >> 1) & 1, vbyte = (c16 & 1) * 8;
          const float rl = lsum > 0.f ? 1.0f / lsum : 0.f;
          const bool store = slot < 2 * S;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) {
            const int piece = dt * 2 + vpiece;
            const s4v lo = lds_tr16(Vb + vr * 256 + ((piece ^ vsw0) << 4) + vbyte);
            const s4v hi = lds_tr16(Vb + (vr + 4) * 256 + ((piece ^ vsw1) << 4) + vbyte);
            const bf16x8 vf = __builtin_bit_cast(bf16x8, (s8v)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            f32x4 o = {0.f, 0.f, 0.f, 0.f};
            o = Mfma<bf16>::mma(vf, pf, o);
            if (store)
              stl8(l2, rw, o_ap + (((i * 2 * S) + slot) * D + 16 * dt + 4 * g) * 2, pack4(o[0] * rl, o[1] * rl, o[2] * rl, o[3] * rl));
          }
          if (store && g == 0)
            stl8(l2, rw, o_am + ((i * 2 * S) + slot) * 8, __builtin_bit_cast(i32x2, make_float2(nk > 0 ? mx : -INFINITY, lsum)));
        }
      }
      leave_group();

      // ================================================================ P3: merge the key chunks
      if (!(alive = enter(Ph<PH_MRG>{}, ls, true))) break;
      {
        const int nvec = 2 * S * (D / 8), per = (nvec + NG - 1) / NG;
        const int v = i * per + (tid >> 3), q = tid & 7;
        const bool act = cw && (tid >> 3) < per;
        const bool valid = act && v < nvec;
        const int vv = valid ? v : 0, slot = vv / (D / 8), dv = vv % (D / 8);
        float2 ml[4];
        i32x4 ov[4];
        if (act) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int ch = 4 * q + c;
            ml[c] = __builtin_bit_cast(float2, ld8(rw, o_am + (ch * 2 * S + slot) * 8));
            ov[c] = ld16(rw, o_ap + ((ch * 2 * S + slot) * D + 8 * dv) * 2);
          }
          float M = -INFINITY;
#pragma unroll
          for (int c = 0; c < 4; ++c) M = fmaxf(M, ml[c].y > 0.f ? ml[c].x : -INFINITY);
          M = max8(M);
          float w[4], Ls = 0.f;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            w[c] = ml[c].y > 0.f ? __builtin_amdgcn_exp2f(ml[c].x - M) * ml[c].y : 0.f;
            Ls += w[c];
          }
          Ls = sum8(Ls);
          float accv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float s = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) s += w[c] > 0.f ? w[c] * bf_to_f(as_bf16x8(ov[c])[e]) : 0.f;
            accv[e] = sum8(s);
          }
          if (valid && q == 0) {
            const float r = Ls > 0.f ? 1.0f / Ls : 0.f;
            bf16x8 o8;
#pragma unroll
            for (int e = 0; e < 8; ++e) o8[e] = (bf16)(accv[e] * r);
            const int qh = slot / S, row = slot - qh * S;
            stl16(l2, rw, o_o + (row * 2 * D + qh * D + 8 * dv) * 2, __builtin_bit_cast(i32x4, o8));
          }
        }
      }
      leave_group();

      // ================================================================ P4: O-projection partial
      if (!(alive = enter(Ph<PH_OPJ>{}, ls, true))) break;
      if (cw) {
        bf16x8 bf[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) bf[u] = bfrag(o_o, 2 * D, 32 * u);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 8; ++u) acc = Mfma<bf16>::mma(afrag(L_O, 32, 16 * hw + c16, u), bf[u], acc);
        const int t = 16 * tt + c16;
        if (t < S) st16(rw, o_opart + ((x * S + t) * H + HC * i + 16 * hw + 4 * g) * 4, tag_bits(acc, ls));
      }
      leave_plain();

      // ================================================================ P5: residual += O-proj
      if (!(alive = enter(Ph<PH_RDO>{}, ls, false))) break;
      if (hown) {
        i32x4 pv[NX];
#pragma unroll
        for (int xx = 0; xx < NX; ++xx) pv[xx] = ld16(rw, o_opart + ((xx * S + ht) * H + hc) * 4);
        poll_tagged(pv, o_opart, ls);
        f32x4 s = __builtin_bit_cast(f32x4, pv[0]);
#pragma unroll
        for (int xx = 1; xx < NX; ++xx) s += __builtin_bit_cast(f32x4, pv[xx]);
        h4 += s;
      }
      publish_h(gain_mlp(l));
      leave_group();

      // ================================================================ P6: gate/up + SwiGLU
      if (!(alive = enter(Ph<PH_GU>{}, ls, true))) break;
      {
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        if (cw) {
          bf16x8 bf[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) bf[u] = bfrag(o_hg, H, 32 * (16 * hw + u));
          const Rms rr = rms_issue();
          const bool rok = c16 < FC;
          const int rg = min(c16, FC - 1), ru = FC + min(c16, FC - 1);
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const int kc = 16 * hw + u;
            bf16x8 ag = afrag(L_GU, 24, rg, kc), au = afrag(L_GU, 24, ru, kc);
            if (!rok) { ag = zero_frag<bf16>(); au = zero_frag<bf16>(); }
            acc0 = Mfma<bf16>::mma(ag, bf[u], acc0);
            acc1 = Mfma<bf16>::mma(au, bf[u], acc1);
          }
          if (hw == 1) {
            *reinterpret_cast<f32x4 *>(smem + L_RED + (tt * 64 + lane) * 16) = acc0;
            *reinterpret_cast<f32x4 *>(smem + L_RED + 4096 + (tt * 64 + lane) * 16) = acc1;
          }
          rms_finish(rr);
        }
        __syncthreads();
        if (cw && hw == 0) {
          acc0 += *reinterpret_cast<const f32x4 *>(smem + L_RED + (tt * 64 + lane) * 16);
          acc1 += *reinterpret_cast<const f32x4 *>(smem + L_RED + 4096 + (tt * 64 + lane) * 16);
          const int t = 16 * tt + c16;
          const float s = inv[min(t, S - 1)];
          if (t < S && g < 3) {  // rows 4g .. 4g+3 < 12: this workgroup's FFN columns
            float y[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] = silu(acc0[j] * s) * (acc1[j] * s);
            stl8(l2, rw, o_act + (t * FG + FC * i + 4 * g) * 2, pack4(y[0], y[1], y[2], y[3]));
          }
        }
      }
      leave_group();

      // ================================================================ P7: down-projection partial
      if (!(alive = enter(Ph<PH_DN>{}, ls, true))) break;
      if (cw) {
        bf16x8 bf[12];
#pragma unroll
        for (int u = 0; u < 12; ++u) bf[u] = bfrag(o_act, FG, 32 * u);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 12; ++u) acc = Mfma<bf16>::mma(afrag(L_D, 32, 16 * hw + c16, u), bf[u], acc);
        const int t = 16 * tt + c16;
        if (t < S) st16(rw, o_dpart + ((x * S + t) * H + HC * i + 16 * hw + 4 * g) * 4, tag_bits(acc, ls));
      }
      leave_plain();

      // ================================================================ P8: residual += down
      if (!(alive = enter(Ph<PH_RDD>{}, ls, false))) break;
      if (hown) {
        i32x4 pv[NX];
#pragma unroll
        for (int xx = 0; xx < NX; ++xx) pv[xx] = ld16(rw, o_dpart + ((xx * S + ht) * H + hc) * 4);
        poll_tagged(pv, o_dpart, ls);
        f32x4 s = __builtin_bit_cast(f32x4, pv[0]);
#pragma unroll
        for (int xx = 1; xx < NX; ++xx) s += __builtin_bit_cast(f32x4, pv[xx]);
        h4 += s;
      }
      if (l + 1 < L) {
        publish_h(gain_attn(l + 1));
      } else {
        // last layer: sums of squares for the final norm, and this slice's share of
        // v[t][a] = sum_c h[t][c] final_norm[c] w_out[a][c] (scaled by 1/rms in the reduce)
        publish_h(nullptr);
        if (hown) {
          const float4 gv = *reinterpret_cast<const float4 *>(gains + 2 * LMAX * HC + (hc - HC * i));
          const float n0 = h4[0] * gv.x, n1 = h4[1] * gv.y, n2 = h4[2] * gv.z, n3 = h4[3] * gv.w;
          for (int q = 0; q < A; ++q) {
            const float4 wv = *reinterpret_cast<const float4 *>(a.w_out + (long)q * H + hc);
            const float s = sum8(n0 * wv.x + n1 * wv.y + n2 * wv.z + n3 * wv.w);
            if ((tid & 7) == 0) stl4f(l2, rw, o_vp + ((i * S + ht) * A + q) * 4, s);
          }
        }
      }
      leave_group();
    }
    if (!alive) break;
    // ================================================================== velocity + Euler
    if (!(alive = enter(Ph<NPH>{}, 0, true))) break;
    if (xown) {
      const int t = xi / A, q = xi - t * A;
      float v = 0.f;
      for (int w = 0; w < NG; ++w) v += ld4f(rw, o_vp + ((w * S + t) * A + q) * 4);
      float ss = 0.f;
      for (int gq = 0; gq < H / 16; gq += 4) {
        const f32x4 u = __builtin_bit_cast(f32x4, ld16(rw, o_ssq + (t * (H / 16) + gq) * 4));
        ss += (u[0] + u[1]) + (u[2] + u[3]);
      }
      v = v * rsqrtf(ss / (float)H + a.eps) + a.b_out[q];
      xv -= v * (1.0f / (float)N);
      stl4f(l2, rw, o_xs + xi * 4, xv);
      if (k == N - 1 && x == 0) a.x[xi] = xv;
    }
    if (k + 1 == N) break;
    leave_group();
    // ================================================================== next step's input
    if (!(alive = enter(Ph<NPH>{}, 0, true))) break;
    embed(k + 1, false);
    publish_h(gain_attn(0));
    leave_group();
  }
  if (!cw) vm_wait<0>();  // no copy may still be landing in LDS when the workgroup ends
  if (!alive && x == 0 && cw) {  // aborted: the chunk is NaN, never a silently wrong value
    for (int e = i * per2 + tid; e < min(S * A, (i + 1) * per2); e += NCW * 64) a.x[e] = NAN;
  }
}

__global__ __launch_bounds__(THREADS) void denoise_b1_kernel(PkArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[L_TOTAL];
  if ((int)(threadIdx.x >> 6) < NCW) pk_run<true>(a, smem);
  else pk_run<false>(a, smem);
}

// Before every launch: zero the sync area and fill the two tagged partial buffers with all-ones
// (epoch tag 3, which the first layer-step, tag 0, does not accept).
__global__ void sync_clear_kernel(int *sync, int n, int *p0, int n0, int *p1, int n1) {
  const int step = gridDim.x * blockDim.x, e0 = blockIdx.x * blockDim.x + threadIdx.x;
  for (int e = e0; e < n; e += step) sync[e] = 0;
  for (int e = e0; e < n0; e += step) p0[e] = -1;
  for (int e = e0; e < n1; e += step) p1[e] = -1;
}

}  // namespace pk

// ---------------------------------------------------------------------------- host side
bool persist_supported(int L, int H, int F, int Hq, int Hkv, int D, int S, int A, int B, int P_cap, bool bf16_dtype) {
  using namespace pk;
  return bf16_dtype && B == 1 && L >= 1 && L <= LMAX && H == pk::H && F == pk::F && Hq == pk::HQ && Hkv == pk::HKV &&
         D == pk::D && S >= 1 && S <= SMAX && A >= 4 && A <= AMAX && A % 4 == 0 && P_cap >= 1 && P_cap <= NG * PC_MAX;
}

size_t persist_ws_bytes(int S, int A) {
  using namespace pk;
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  size_t t = 0;
  t += up((size_t)NX * S * H * 2);           // hg
  t += up((size_t)NX * S * (H / 16) * 4);    // ssq
  t += up((size_t)NX * S * GW * 2);          // qkv
  t += up((size_t)NX * NG * 2 * S * D * 2);  // apart
  t += up((size_t)NX * NG * 2 * S * 8);      // aml
  t += up((size_t)NX * S * 2 * D * 2);       // o
  t += up((size_t)NX * S * H * 4);           // opart
  t += up((size_t)NX * S * FG * 2);          // act
  t += up((size_t)NX * S * H * 4);           // dpart
  t += up((size_t)NX * NG * S * A * 4);      // vpart
  t += up((size_t)NX * S * A * 4);           // xs
  t += up((size_t)SYNC_INTS * 4);            // sync
  return t;
}

hipError_t launch_denoise_persistent(const PersistLaunch &p, hipStream_t s) {
  using namespace pk;
  PkArgs a;
  a.w_qkv = (const bf16 *)p.w_qkv; a.w_o = (const bf16 *)p.w_o; a.w_gate = (const bf16 *)p.w_gate;
  a.w_up = (const bf16 *)p.w_up; a.w_down = (const bf16 *)p.w_down;
  a.attn_norm = p.attn_norm; a.mlp_norm = p.mlp_norm;
  a.w_in = p.w_in; a.b_in = p.b_in; a.final_norm = p.final_norm; a.w_out = p.w_out; a.b_out = p.b_out;
  a.k_cache = (const bf16 *)p.k_cache; a.v_cache = (const bf16 *)p.v_cache; a.lens = p.lens; a.x = p.x;
  a.L = p.L; a.S = p.S; a.A = p.A; a.P_cap = p.P_cap; a.steps = p.steps; a.eps = p.eps; a.rope_base = p.rope_base;
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const int S = p.S, A = p.A;
  size_t w = 0;
  auto put = [&](int &off, size_t bytes) { off = (int)w; w += up(bytes); };
  put(a.off_hg, (size_t)NX * S * H * 2);
  put(a.off_ssq, (size_t)NX * S * (H / 16) * 4);
  put(a.off_qkv, (size_t)NX * S * GW * 2);
  put(a.off_apart, (size_t)NX * NG * 2 * S * D * 2);
  put(a.off_aml, (size_t)NX * NG * 2 * S * 8);
  put(a.off_o, (size_t)NX * S * 2 * D * 2);
  put(a.off_opart, (size_t)NX * S * H * 4);
  put(a.off_act, (size_t)NX * S * FG * 2);
  put(a.off_dpart, (size_t)NX * S * H * 4);
  put(a.off_vpart, (size_t)NX * NG * S * A * 4);
  put(a.off_xs, (size_t)NX * S * A * 4);
  a.ws_base = (char *)p.ws;
  a.ws_bytes = (int)w;
  a.sync = (int *)((char *)p.ws + w);
  hipLaunchKernelGGL(sync_clear_kernel, dim3(256), dim3(256), 0, s, a.sync, (int)SYNC_INTS,
                     (int *)(a.ws_base + a.off_opart), NX * S * H, (int *)(a.ws_base + a.off_dpart), NX * S * H);
  hipLaunchKernelGGL(denoise_b1_kernel, dim3(NWG), dim3(THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t persist_check_device(int device) {
  int cus = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return e;
  int occ = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, pk::denoise_b1_kernel, pk::THREADS, 0);
  if (e != hipSuccess) return e;
  return (cus >= pk::NWG && occ >= 1) ? hipSuccess : hipErrorInvalidConfiguration;
}

}  // namespace dm

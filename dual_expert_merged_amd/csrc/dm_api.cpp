// C ABI of libdm: argument validation, workspace layout, and the launch sequences of the three
// operations (prefix encoding, one merged layer, suffix denoising) plus hipGraph plans.
// What each call computes is documented with its declaration in include/dm.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <new>
#include <string>

#include "../../include/dm.h"
#include "kernels.h"

using namespace dm;

namespace {

thread_local std::string g_err;

dm_status fail(dm_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

#define REQUIRE(cond, st, ...) \
  do {                         \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

#define HIP_TRY(expr)                                                                          \
  do {                                                                                         \
    hipError_t e_ = (expr);                                                                    \
    if (e_ != hipSuccess) return fail(DM_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_));   \
  } while (0)

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

struct dm_ctx {
  dm_config cfg;
  int device;
  Dt dt;
  size_t es;  // bytes per element of the weight dtype
};

struct dm_plan {
  hipGraph_t graph;
  hipGraphExec_t exec;
  int steps;
  int device;
};

// ----------------------------------------------------------------------------- workspace layout

namespace {

struct Region {
  size_t off = 0, bytes = 0;
};

// Tile plans of the GEMMs of one expert at one row count.
struct ExpertPlans {
  GemmPlan qkv, o, gu, down;
};

struct Layout {
  Region rope, rope_rows;
  Region h, hg, ssq, q, ks, vs, o, act, apart, split;          // action side (h: denoise only)
  Region hp, hg_p, ssq_p, q_p, kp, vp, o_p, act_p, apart_p;    // prefix side (hp: prefill only)
  Region q8_p, qs_p;                                           // FP8 MLP operand codes and row scales
  int n_chunks = 1, chunk_keys = 32, n_chunks_p = 1, chunk_keys_p = 32;
  ExpertPlans pa, pv;  // action expert, VLM expert
  size_t total = 0;
  void put(Region &r, size_t bytes) {
    r.off = total;
    r.bytes = bytes;
    total += up256(bytes);
  }
};

void attn_split(int B, int Hkv, int nqb, int max_keys, int *n_chunks, int *chunk_keys) {
  const int blocks = B * Hkv * nqb;
  // as many chunks as still fit one round of workgroups on the 256 CUs (one per CU): a partial
  // second round costs more than the longer chunks (one merged layer's prefix attention, 104
  // groups: 3 chunks 24.5 + 9.2 us merge)
  int want = 256 / blocks;
  if (want > 16) want = 16;  // the merge keeps every chunk's statistics in registers
  const int maxc = (max_keys + 63) / 64;  // at least one 64-key tile per chunk
  if (want > maxc) want = maxc;
  if (want < 1) want = 1;
  int ck = (max_keys + want - 1) / want;
  ck = (ck + 31) / 32 * 32;
  *chunk_keys = ck;
  *n_chunks = (max_keys + ck - 1) / ck;
}

// M <= 64 rows: the skinny kernel.  Every workgroup takes 32 output columns (each re-reads the
// whole activation slice from L2, so wider tiles cut that traffic); narrow GEMMs (the residual
// projections) also split K until ~256 workgroups.
// Each wave of the skinny kernel holds its whole K slice in registers: at most 8 MFMA k-chunks,
// otherwise K is split further (residual projections) or the tiled kernel is used.
GemmPlan plan_gemm(Dt dt, int M, int N, int K, bool split_ok) {
  GemmPlan p{};
  p.sk.k_split = 1;
  p.skinny = 0;
  p.nt = 0;  // the tiled kernel
  if (M > 64) {
    // bf16: 128-row tiles, 256 columns when that still gives >= 128 workgroups, else 128; narrow
    // GEMMs take 64 columns, or split K (multiples of 64) until ~200 workgroups.
    if (dt != DT_BF16 || N % 128 != 0 || K % 64 != 0) return p;
    if (N % 256 == 0 && (size_t)(N / 256) * ((M + 255) / 256) >= 200) {
      // 256 x 256 tiles while they still make ~200 workgroups (the prefill shapes: a third fewer
      // copied bytes per MFMA than 128 x 384, 4-14 % faster there; fewer workgroups lose)
      p.nt = 256;
      p.bm = 256;
      return p;
    }
    const int mt = (M + 127) / 128;
    if (split_ok && N % 64 == 0 && (N / 64) * mt >= 200) {
      // residual projections: 128 x 64 tiles fill the CUs without a K split, so the residual
      // epilogue runs in the same launch (batch 32, O: 18.1 -> 16.7 us with the reduce)
      p.nt = 64;
      return p;
    }
    p.nt = (N % 256 == 0 && (N / 256) * mt >= 128) ? 256 : 128;
    if (!split_ok && p.nt == 256 && N % 384 == 0) {
      // one workgroup per CU: compare whole rounds of 256 workgroups, a 384-wide tile costing
      // about 1.5 times a 256-wide one
      const int r256 = ((N / 256) * mt + 255) / 256, r384 = ((N / 384) * mt + 255) / 256;
      if (2 * r384 * 3 < 2 * r256 * 2) p.nt = 384;
    }
    if (split_ok)
      while ((N / p.nt) * mt * p.sk.k_split < 200 && p.sk.k_split < 8 && K % (2 * p.sk.k_split * 64) == 0 &&
             K / (2 * p.sk.k_split) >= 256)
        p.sk.k_split *= 2;
    return p;
  }
  const int kq = gemm_k_quantum(dt);  // K per k-chunk across the 4 waves
  if (split_ok && N % 16 == 0 && K % (4 * kq) == 0 && K / (4 * kq) <= 8 && (N / 16) * ((M + 15) / 16) >= 128) {
    // residual projections: 16 waves per workgroup cover the whole K of 16 columns x 16 rows,
    // enough workgroups without a K split, so the residual epilogue runs in the same launch
    // (batch 1, O: 7.7 -> 6.7 us in isolation, one launch fewer)
    p.skinny = 1;
    p.nt = 16;
    p.rt = 1;
    p.nw = 16;
    return p;
  }
  const int nt = N % 32 == 0 ? 32 : 16;
  int ks = 1;
  if (split_ok) {
    while ((N / nt) * ks < 256 && ks < 16 && K % (2 * ks * kq) == 0) ks *= 2;
    while (K / (ks * kq) > 8 && ks < 16 && K % (2 * ks * kq) == 0) ks *= 2;
  }
  if (K % (ks * kq) != 0 || K / (ks * kq) > 8) return p;
  p.skinny = 1;
  p.nt = nt;
  p.sk.k_split = ks;
  // half-height workgroups when twice as many still fit the 256 CUs in one round: each reads
  // half the activation rows, and twice the CUs pull the weights (QKV at batch 1: 9.2 -> 7.5 us)
  if (M > 32 && (size_t)(N / nt) * ks * ((M + 31) / 32) <= 256) p.rt = 2;
  return p;
}

ExpertPlans plan_expert(const dm_config &c, Dt dt, int M, int H, int F) {
  ExpertPlans e;
  const int QKV = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim, QD = c.n_q_heads * c.head_dim;
  e.qkv = plan_gemm(dt, M, QKV, H, false);
  e.o = plan_gemm(dt, M, H, QD, true);
  e.gu = plan_gemm(dt, M, 2 * F, H, false);
  e.down = plan_gemm(dt, M, H, F, true);
  return e;
}

size_t split_bytes(const GemmPlan &p, int M, int N) {
  return p.sk.k_split > 1 ? (size_t)p.sk.k_split * M * N * sizeof(float) : 0;
}

Layout make_layout(const dm_config &c, size_t es, dm_op op, int B, int P_cap) {
  Layout L;
  const Dt dt = es == 2 ? DT_BF16 : DT_F32;
  const int S = c.chunk, D = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
  const int Ha = c.act_hidden, Hv = c.vlm_hidden;
  const size_t Ms = (size_t)B * S, Mp = (size_t)B * P_cap;
  L.put(L.rope, (size_t)(P_cap + S) * (D / 2) * sizeof(float2));
  if (op != DM_OP_PREFILL) L.put(L.rope_rows, (size_t)B * S * (D / 2) * sizeof(float2));
  size_t split = 0;
  if (op == DM_OP_DENOISE || op == DM_OP_MERGED_LAYER) {
    L.pa = plan_expert(c, dt, (int)Ms, Ha, c.act_ffn);
    split = std::max(split_bytes(L.pa.o, (int)Ms, Ha), split_bytes(L.pa.down, (int)Ms, Ha));
    if (op == DM_OP_DENOISE) L.put(L.h, Ms * Ha * sizeof(float));
    L.put(L.hg, Ms * Ha * es);
    L.put(L.ssq, Ms * (Ha / 16) * sizeof(float));
    L.put(L.q, Ms * Hq * D * es);
    L.put(L.ks, (size_t)B * Hkv * S * D * es);
    L.put(L.vs, (size_t)B * Hkv * S * D * es);
    L.put(L.o, Ms * Hq * D * es);
    L.put(L.act, Ms * c.act_ffn * es);
    const int nqb = attn_qblocks(S, Hq, Hkv);
    attn_split(B, Hkv, nqb, P_cap + S, &L.n_chunks, &L.chunk_keys);
    if (L.n_chunks > 1) L.put(L.apart, attn_partial_bytes(dt, B, Hkv, nqb, L.n_chunks, D));
  }
  if (op == DM_OP_PREFILL || op == DM_OP_MERGED_LAYER) {
    L.pv = plan_expert(c, dt, (int)Mp, Hv, c.vlm_ffn);
    split = std::max(split, std::max(split_bytes(L.pv.o, (int)Mp, Hv), split_bytes(L.pv.down, (int)Mp, Hv)));
    if (op == DM_OP_PREFILL) L.put(L.hp, Mp * Hv * sizeof(float));
    L.put(L.hg_p, Mp * Hv * es);
    L.put(L.ssq_p, Mp * (Hv / 16) * sizeof(float));
    L.put(L.q_p, Mp * Hq * D * es);
    if (op == DM_OP_MERGED_LAYER) {
      L.put(L.kp, (size_t)B * Hkv * P_cap * D * es);
      L.put(L.vp, (size_t)B * Hkv * P_cap * D * es);
    }
    L.put(L.o_p, Mp * Hq * D * es);
    L.put(L.act_p, Mp * c.vlm_ffn * es);
    if (op == DM_OP_PREFILL && c.vlm_mlp_dtype == DM_FP8_E4M3) {
      L.put(L.q8_p, Mp * (size_t)std::max(Hv, c.vlm_ffn));
      L.put(L.qs_p, Mp * sizeof(float));
    }
    const int nqb = attn_qblocks(P_cap, Hq, Hkv);
    attn_split(B, Hkv, nqb, P_cap, &L.n_chunks_p, &L.chunk_keys_p);
    if (L.n_chunks_p > 1) L.put(L.apart_p, attn_partial_bytes(dt, B, Hkv, nqb, L.n_chunks_p, D));
  }
  if (split) L.put(L.split, split);
  return L;
}

template <typename P> P *at(void *ws, const Region &r) { return (P *)((char *)ws + r.off); }

dm_status check_config(const dm_config *c) {
  REQUIRE(c, DM_ERR_INVALID_ARG, "config is NULL");
  REQUIRE(c->dtype == DM_F32 || c->dtype == DM_BF16, DM_ERR_UNSUPPORTED, "dtype must be DM_F32 or DM_BF16");
  REQUIRE(c->vlm_mlp_dtype == c->dtype || (c->vlm_mlp_dtype == DM_FP8_E4M3 && c->dtype == DM_BF16),
          DM_ERR_UNSUPPORTED, "vlm_mlp_dtype must equal dtype, or be DM_FP8_E4M3 with DM_BF16");
  REQUIRE(c->n_layers >= 1, DM_ERR_SHAPE, "n_layers must be >= 1");
  REQUIRE(c->head_dim == 32 || c->head_dim == 64 || c->head_dim == 128, DM_ERR_UNSUPPORTED,
          "head_dim must be 32, 64 or 128");
  REQUIRE(c->n_kv_heads >= 1 && c->n_q_heads >= c->n_kv_heads && c->n_q_heads % c->n_kv_heads == 0, DM_ERR_SHAPE,
          "n_q_heads must be a multiple of n_kv_heads");
  const int g = c->n_q_heads / c->n_kv_heads;
  REQUIRE(g == 1 || g == 2 || g == 4, DM_ERR_UNSUPPORTED, "query heads per KV head must be 1, 2 or 4");
  REQUIRE(c->vlm_hidden > 0 && c->vlm_hidden % 64 == 0 && c->act_hidden > 0 && c->act_hidden % 64 == 0, DM_ERR_SHAPE,
          "hidden sizes must be positive multiples of 64");
  REQUIRE(c->vlm_ffn > 0 && c->vlm_ffn % 64 == 0 && c->act_ffn > 0 && c->act_ffn % 64 == 0, DM_ERR_SHAPE,
          "FFN sizes must be positive multiples of 64");
  REQUIRE((c->n_q_heads * c->head_dim) % 64 == 0, DM_ERR_SHAPE, "n_q_heads*head_dim must be a multiple of 64");
  REQUIRE(((c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim) % 64 == 0, DM_ERR_SHAPE,
          "(n_q_heads+2*n_kv_heads)*head_dim must be a multiple of 64");
  const int kq = c->dtype == DM_BF16 ? 128 : 64;  // one K step of the skinny kernel (4 waves x one MFMA chunk)
  REQUIRE(c->vlm_hidden % kq == 0 && c->act_hidden % kq == 0 && (c->n_q_heads * c->head_dim) % kq == 0 &&
              c->vlm_ffn % kq == 0 && c->act_ffn % kq == 0,
          DM_ERR_SHAPE, "hidden, FFN and n_q_heads*head_dim must be multiples of %d for this dtype", kq);
  REQUIRE(c->vlm_hidden <= 4096 && c->act_hidden <= 4096, DM_ERR_UNSUPPORTED, "hidden sizes above 4096");
  REQUIRE(c->vlm_mlp_dtype != DM_FP8_E4M3 || (c->vlm_hidden % 128 == 0 && c->vlm_ffn % 128 == 0), DM_ERR_SHAPE,
          "the FP8 MLP needs vlm_hidden and vlm_ffn to be multiples of 128");
  REQUIRE(c->action_dim >= 4 && c->action_dim <= 64 && c->action_dim % 4 == 0, DM_ERR_UNSUPPORTED,
          "action_dim must be a multiple of 4 in 4..64");
  REQUIRE(c->chunk >= 1 && c->chunk <= 64, DM_ERR_UNSUPPORTED, "chunk must be 1..64");
  REQUIRE(c->rms_eps > 0.f && std::isfinite(c->rms_eps), DM_ERR_INVALID_ARG, "rms_eps must be positive");
  REQUIRE(c->rope_base > 1.f && std::isfinite(c->rope_base), DM_ERR_INVALID_ARG, "rope_base must be > 1");
  return DM_OK;
}

dm_status check_expert(const dm_expert_weights *w, bool fp8, const char *name) {
  REQUIRE(w, DM_ERR_INVALID_ARG, "%s weights are NULL", name);
  const void *ptrs[] = {w->attn_norm, w->w_qkv, w->w_o, w->mlp_norm, w->w_gate, w->w_up, w->w_down};
  for (const void *p : ptrs) {
    REQUIRE(p, DM_ERR_INVALID_ARG, "%s weights: a tensor pointer is NULL", name);
    REQUIRE(aligned16(p), DM_ERR_INVALID_ARG, "%s weights: a tensor pointer is not 16-byte aligned", name);
  }
  if (fp8) {
    REQUIRE(w->s_gate && w->s_up && w->s_down, DM_ERR_INVALID_ARG, "%s weights: FP8 MLP needs s_gate/s_up/s_down",
            name);
  }
  return DM_OK;
}

dm_status check_common(const dm_ctx *ctx, const int32_t *lens, int B, int P_cap, void *ws, size_t ws_bytes,
                       dm_op op) {
  REQUIRE(ctx, DM_ERR_INVALID_ARG, "ctx is NULL");
  REQUIRE(lens, DM_ERR_INVALID_ARG, "prefix_lens is NULL");
  REQUIRE(B >= 1 && B <= 4096, DM_ERR_SHAPE, "B must be 1..4096 (got %d)", B);
  REQUIRE(P_cap >= 1 && P_cap <= 65536, DM_ERR_SHAPE, "P_cap must be 1..65536 (got %d)", P_cap);
  REQUIRE(ws, DM_ERR_INVALID_ARG, "workspace is NULL");
  REQUIRE(((uintptr_t)ws & 255u) == 0, DM_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const size_t need = make_layout(ctx->cfg, ctx->es, op, B, P_cap).total;
  REQUIRE(ws_bytes >= need, DM_ERR_WORKSPACE, "workspace too small: %zu bytes, need %zu", ws_bytes, need);
  return DM_OK;
}

#define TRY(expr)                    \
  do {                               \
    dm_status s_ = (expr);           \
    if (s_ != DM_OK) return s_;      \
  } while (0)

const char *layer_ptr(const void *base, size_t layer_elems, int l, size_t es) {
  return (const char *)base + (size_t)l * layer_elems * es;
}

// ----------------------------------------------------------------------------- launch sequences

struct Expert {
  const float *attn_norm, *mlp_norm;
  const void *w_qkv, *w_o, *w_gate, *w_up, *w_down;
  const float *s_gate = nullptr, *s_up = nullptr, *s_down = nullptr;  // FP8 MLP only
};

// Layer l of a stacked expert; fp8: the MLP matrices are one-byte E4M3 codes with scales.
Expert expert_layer(const dm_config &c, const dm_expert_weights &w, int l, int H, int F, size_t es,
                    bool fp8 = false) {
  const int QKV = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim, QD = c.n_q_heads * c.head_dim;
  const size_t mes = fp8 ? 1 : es;
  Expert e;
  e.attn_norm = w.attn_norm + (size_t)l * H;
  e.mlp_norm = w.mlp_norm + (size_t)l * H;
  e.w_qkv = layer_ptr(w.w_qkv, (size_t)QKV * H, l, es);
  e.w_o = layer_ptr(w.w_o, (size_t)H * QD, l, es);
  e.w_gate = layer_ptr(w.w_gate, (size_t)F * H, l, mes);
  e.w_up = layer_ptr(w.w_up, (size_t)F * H, l, mes);
  e.w_down = layer_ptr(w.w_down, (size_t)H * F, l, mes);
  if (fp8) {
    e.s_gate = w.s_gate + (size_t)l * F;
    e.s_up = w.s_up + (size_t)l * F;
    e.s_down = w.s_down + (size_t)l * H;
  }
  return e;
}

SplitK splitk(const Layout &L, void *ws, const GemmPlan &p) {
  SplitK s = p.sk;
  s.part = L.split.bytes ? at<float>(ws, L.split) : nullptr;
  return s;
}

// One expert's O-projection + residual and MLP + residual.  `next_attn_norm` is the gain of
// the norm that follows the layer (NULL after the last layer of a stack).
void enqueue_finish(const dm_ctx *ctx, const Layout &L, void *ws, const ExpertPlans &pl, const Expert &e,
                    const Hidden &hid, const void *o, void *act, int M, int F, RowMap rows,
                    const float *next_attn_norm, hipStream_t s) {
  const dm_config &c = ctx->cfg;
  GemmPlan po = pl.o, pg = pl.gu, pd = pl.down;
  po.sk = splitk(L, ws, pl.o);
  pd.sk = splitk(L, ws, pl.down);
  ResidArgs ro{o, M, c.n_q_heads * c.head_dim, e.w_o, hid, e.mlp_norm, rows};
  launch_resid(ctx->dt, ro, po, s);
  SwigluArgs sg{hid, M, F, c.rms_eps, e.w_gate, e.w_up, act, rows};
  launch_swiglu(ctx->dt, sg, pg, s);
  ResidArgs rd{act, M, F, e.w_down, hid, next_attn_norm, rows};
  launch_resid(ctx->dt, rd, pd, s);
}

// The same with the MLP in FP8 E4M3 (page "DM0.5: High-Performance Embodied VLA ...", section
// 6.3): the normalised MLP input and the SwiGLU activation are quantised per token, the three
// MLP GEMMs run on FP8 MFMA with fp32 accumulation, scales applied in the epilogues.
void enqueue_finish_fp8(const dm_ctx *ctx, const Layout &L, void *ws, const ExpertPlans &pl, const Expert &e,
                        const Hidden &hid, const void *o, void *act, int M, int F, RowMap rows,
                        const float *next_attn_norm, hipStream_t s) {
  const dm_config &c = ctx->cfg;
  GemmPlan po = pl.o;
  po.sk = splitk(L, ws, pl.o);
  ResidArgs ro{o, M, c.n_q_heads * c.head_dim, e.w_o, hid, e.mlp_norm, rows};
  launch_resid(ctx->dt, ro, po, s);
  uint8_t *q8 = at<uint8_t>(ws, L.q8_p);
  float *qs = at<float>(ws, L.qs_p);
  launch_fp8_quantize_rows(hid.hg, q8, qs, M, hid.H, s);
  SwigluArgs sg{hid, M, F, c.rms_eps, e.w_gate, e.w_up, act, rows, q8, qs, e.s_gate, e.s_up};
  launch_swiglu_fp8(sg, s);
  launch_fp8_quantize_rows(act, q8, qs, M, F, s);
  ResidArgs rd{q8, M, F, e.w_down, hid, next_attn_norm, rows, qs, e.s_down};
  launch_resid_fp8(rd, s);
}

dm_status enqueue_denoise(const dm_ctx *ctx, const dm_action_weights *aw, const void *k_cache, const void *v_cache,
                          const int32_t *lens, int B, int P_cap, float *x, int num_steps, void *ws, hipStream_t s) {
  const dm_config &c = ctx->cfg;
  const Layout L = make_layout(c, ctx->es, DM_OP_DENOISE, B, P_cap);
  const int S = c.chunk, Ha = c.act_hidden, Fa = c.act_ffn, D = c.head_dim, Hkv = c.n_kv_heads;
  const int M = B * S;
  float2 *rope = at<float2>(ws, L.rope);
  const Hidden hid{at<float>(ws, L.h), at<void>(ws, L.hg), at<float>(ws, L.ssq), Ha};
  void *q = at<void>(ws, L.q), *ks = at<void>(ws, L.ks), *vs = at<void>(ws, L.vs);
  void *o = at<void>(ws, L.o), *act = at<void>(ws, L.act);
  const RowMap rows{S, lens, 0, P_cap};
  const size_t layer_cache = (size_t)B * Hkv * P_cap * D;
  const GemmPlan pq = L.pa.qkv;

  launch_rope_table(rope, P_cap + S, D, c.rope_base, s);
  float2 *rope_rows = at<float2>(ws, L.rope_rows);
  launch_rope_rows(rope, lens, P_cap, B, S, D, rope_rows, s);
  for (int k = 0; k < num_steps; ++k) {
    const float t = 1.0f - (float)k / (float)num_steps;
    launch_embed(ctx->dt, x, aw->w_in, aw->b_in, hid, aw->body.attn_norm, M, c.action_dim, t, s);
    for (int l = 0; l < c.n_layers; ++l) {
      const Expert e = expert_layer(c, aw->body, l, Ha, Fa, ctx->es);
      QkvArgs qa{hid, M, c.rms_eps, e.w_qkv, q, ks, vs, S, rows, rope, c.n_q_heads, Hkv, D, rope_rows};
      launch_qkv(ctx->dt, qa, pq, s);
      AttnArgs aa{q, S, 1,
                  layer_ptr(k_cache, layer_cache, l, ctx->es), layer_ptr(v_cache, layer_cache, l, ctx->es), P_cap,
                  ks, vs, S, lens, B, c.n_q_heads, Hkv, D, L.n_chunks, L.chunk_keys, o,
                  L.n_chunks > 1 ? at<void>(ws, L.apart) : nullptr};
      launch_attention(ctx->dt, aa, s);
      const float *next = l + 1 < c.n_layers ? aw->body.attn_norm + (size_t)(l + 1) * Ha : nullptr;
      enqueue_finish(ctx, L, ws, L.pa, e, hid, o, act, M, Fa, rows, next, s);
    }
    launch_velocity_euler(hid.h, aw->final_norm, aw->w_out, aw->b_out, x, M, Ha, c.action_dim, c.rms_eps, num_steps,
                          s);
  }
  return DM_OK;
}

dm_status check_action(const dm_ctx *ctx, const dm_action_weights *aw) {
  REQUIRE(aw, DM_ERR_INVALID_ARG, "action weights are NULL");
  TRY(check_expert(&aw->body, false, "action"));
  const void *ptrs[] = {aw->w_in, aw->b_in, aw->final_norm, aw->w_out, aw->b_out};
  for (const void *p : ptrs) {
    REQUIRE(p, DM_ERR_INVALID_ARG, "action head: a tensor pointer is NULL");
    REQUIRE(aligned16(p), DM_ERR_INVALID_ARG, "action head: a tensor pointer is not 16-byte aligned");
  }
  (void)ctx;
  return DM_OK;
}

dm_status check_denoise(dm_ctx *ctx, const dm_action_weights *aw, const void *k_cache, const void *v_cache,
                        const int32_t *lens, int B, int P_cap, float *x, int num_steps, void *ws, size_t ws_bytes) {
  TRY(check_common(ctx, lens, B, P_cap, ws, ws_bytes, DM_OP_DENOISE));
  TRY(check_action(ctx, aw));
  REQUIRE(k_cache && v_cache, DM_ERR_INVALID_ARG, "k_cache / v_cache is NULL");
  REQUIRE(aligned16(k_cache) && aligned16(v_cache), DM_ERR_INVALID_ARG, "caches must be 16-byte aligned");
  REQUIRE(x, DM_ERR_INVALID_ARG, "x is NULL");
  REQUIRE(aligned16(x), DM_ERR_INVALID_ARG, "x must be 16-byte aligned");
  REQUIRE(num_steps >= 1 && num_steps <= 1000, DM_ERR_SHAPE, "num_steps must be 1..1000 (got %d)", num_steps);
  return DM_OK;
}

dm_status set_device(const dm_ctx *ctx) {
  int cur = -1;
  HIP_TRY(hipGetDevice(&cur));
  if (cur != ctx->device) HIP_TRY(hipSetDevice(ctx->device));
  return DM_OK;
}

}  // namespace

// ============================================================================= exported C ABI

extern "C" {

const char *dm_version(void) { return "libdm 0.1 (gfx950)"; }

const char *dm_last_error(void) { return g_err.c_str(); }

dm_status dm_ctx_create(const dm_config *cfg, int device, dm_ctx **out) {
  REQUIRE(out, DM_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  TRY(check_config(cfg));
  REQUIRE(device >= 0, DM_ERR_INVALID_ARG, "device must be >= 0");
  int n = 0;
  HIP_TRY(hipGetDeviceCount(&n));
  REQUIRE(device < n, DM_ERR_INVALID_ARG, "device %d out of range (%d devices)", device, n);
  dm_ctx *ctx = new (std::nothrow) dm_ctx;
  REQUIRE(ctx, DM_ERR_INVALID_ARG, "out of host memory");
  ctx->cfg = *cfg;
  ctx->device = device;
  ctx->dt = cfg->dtype == DM_BF16 ? DT_BF16 : DT_F32;
  ctx->es = cfg->dtype == DM_BF16 ? 2 : 4;
  *out = ctx;
  return DM_OK;
}

void dm_ctx_destroy(dm_ctx *ctx) { delete ctx; }

size_t dm_workspace_bytes(const dm_ctx *ctx, dm_op op, int B, int P_cap) {
  if (!ctx || B < 1 || P_cap < 1 || (op != DM_OP_PREFILL && op != DM_OP_MERGED_LAYER && op != DM_OP_DENOISE)) return 0;
  return make_layout(ctx->cfg, ctx->es, op, B, P_cap).total;
}

dm_status dm_suffix_denoise(dm_ctx *ctx, const dm_action_weights *aw, const void *k_cache, const void *v_cache,
                            const int32_t *prefix_lens, int B, int P_cap, float *x, int num_steps, void *ws,
                            size_t ws_bytes, void *stream) {
  TRY(check_denoise(ctx, aw, k_cache, v_cache, prefix_lens, B, P_cap, x, num_steps, ws, ws_bytes));
  TRY(set_device(ctx));
  hipStream_t s = (hipStream_t)stream;
  TRY(enqueue_denoise(ctx, aw, k_cache, v_cache, prefix_lens, B, P_cap, x, num_steps, ws, s));
  HIP_TRY(hipGetLastError());
  return DM_OK;
}

dm_status dm_denoise_plan_create(dm_ctx *ctx, const dm_action_weights *aw, const void *k_cache, const void *v_cache,
                                 const int32_t *prefix_lens, int B, int P_cap, float *x, int num_steps, void *ws,
                                 size_t ws_bytes, void *stream, dm_plan **out) {
  REQUIRE(out, DM_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  TRY(check_denoise(ctx, aw, k_cache, v_cache, prefix_lens, B, P_cap, x, num_steps, ws, ws_bytes));
  TRY(set_device(ctx));
  hipStream_t cs = nullptr;
  HIP_TRY(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking));
  hipGraph_t graph = nullptr;
  hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeRelaxed);
  if (e != hipSuccess) {
    (void)hipStreamDestroy(cs);
    return fail(DM_ERR_HIP, "hipStreamBeginCapture: %s", hipGetErrorString(e));
  }
  enqueue_denoise(ctx, aw, k_cache, v_cache, prefix_lens, B, P_cap, x, num_steps, ws, cs);
  e = hipStreamEndCapture(cs, &graph);
  (void)hipStreamDestroy(cs);
  if (e != hipSuccess) return fail(DM_ERR_HIP, "hipStreamEndCapture: %s", hipGetErrorString(e));
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return fail(DM_ERR_HIP, "hipGraphInstantiate: %s", hipGetErrorString(e));
  }
  e = hipGraphUpload(exec, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    return fail(DM_ERR_HIP, "hipGraphUpload: %s", hipGetErrorString(e));
  }
  dm_plan *p = new (std::nothrow) dm_plan{graph, exec, num_steps, ctx->device};
  if (!p) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    return fail(DM_ERR_INVALID_ARG, "out of host memory");
  }
  *out = p;
  return DM_OK;
}

dm_status dm_denoise_plan_launch(dm_plan *plan, int num_steps, void *stream) {
  REQUIRE(plan, DM_ERR_INVALID_ARG, "plan is NULL");
  REQUIRE(num_steps == plan->steps, DM_ERR_PLAN_MISMATCH,
          "num_steps %d differs from the %d steps captured in the plan", num_steps, plan->steps);
  HIP_TRY(hipGraphLaunch(plan->exec, (hipStream_t)stream));
  return DM_OK;
}

void dm_denoise_plan_destroy(dm_plan *plan) {
  if (!plan) return;
  (void)hipGraphExecDestroy(plan->exec);
  (void)hipGraphDestroy(plan->graph);
  delete plan;
}

dm_status dm_merged_layer(dm_ctx *ctx, const dm_expert_weights *vlm, const dm_expert_weights *act, int layer,
                          float *h_prefix, float *h_suffix, const int32_t *prefix_lens, int B, int P_cap, void *k_out,
                          void *v_out, void *ws, size_t ws_bytes, void *stream) {
  TRY(check_common(ctx, prefix_lens, B, P_cap, ws, ws_bytes, DM_OP_MERGED_LAYER));
  const dm_config &c = ctx->cfg;
  REQUIRE(c.vlm_mlp_dtype == c.dtype, DM_ERR_UNSUPPORTED, "dm_merged_layer runs the VLM MLP in the weight dtype");
  TRY(check_expert(vlm, false, "VLM"));
  TRY(check_expert(act, false, "action"));
  REQUIRE(layer >= 0 && layer < c.n_layers, DM_ERR_SHAPE, "layer %d out of range", layer);
  REQUIRE(h_prefix && h_suffix, DM_ERR_INVALID_ARG, "h_prefix / h_suffix is NULL");
  REQUIRE(aligned16(h_prefix) && aligned16(h_suffix), DM_ERR_INVALID_ARG, "hidden streams must be 16-byte aligned");
  REQUIRE((k_out == nullptr) == (v_out == nullptr), DM_ERR_INVALID_ARG, "k_out and v_out must both be set or NULL");
  REQUIRE(!k_out || (aligned16(k_out) && aligned16(v_out)), DM_ERR_INVALID_ARG, "k_out / v_out must be aligned");
  TRY(set_device(ctx));
  hipStream_t s = (hipStream_t)stream;
  const Layout L = make_layout(c, ctx->es, DM_OP_MERGED_LAYER, B, P_cap);
  const int S = c.chunk, D = c.head_dim, Hkv = c.n_kv_heads, Hq = c.n_q_heads;
  const int Ms = B * S, Mp = B * P_cap;
  float2 *rope = at<float2>(ws, L.rope);
  void *kp = k_out ? k_out : at<void>(ws, L.kp), *vp = v_out ? v_out : at<void>(ws, L.vp);
  const RowMap prow{P_cap, prefix_lens, 1, P_cap}, srow{S, prefix_lens, 0, P_cap};
  const Expert ev = expert_layer(c, *vlm, layer, c.vlm_hidden, c.vlm_ffn, ctx->es);
  const Expert ea = expert_layer(c, *act, layer, c.act_hidden, c.act_ffn, ctx->es);
  const Hidden hp{h_prefix, at<void>(ws, L.hg_p), at<float>(ws, L.ssq_p), c.vlm_hidden};
  const Hidden hs{h_suffix, at<void>(ws, L.hg), at<float>(ws, L.ssq), c.act_hidden};

  launch_rope_table(rope, P_cap + S, D, c.rope_base, s);
  float2 *rope_rows = at<float2>(ws, L.rope_rows);
  launch_rope_rows(rope, prefix_lens, P_cap, B, S, D, rope_rows, s);
  launch_norm_prep(ctx->dt, h_prefix, hp, ev.attn_norm, Mp, s);
  launch_norm_prep(ctx->dt, h_suffix, hs, ea.attn_norm, Ms, s);
  QkvArgs qv{hp, Mp, c.rms_eps, ev.w_qkv, at<void>(ws, L.q_p), kp, vp, P_cap, prow, rope, Hq, Hkv, D};
  launch_qkv(ctx->dt, qv, L.pv.qkv, s);
  QkvArgs qa{hs, Ms, c.rms_eps, ea.w_qkv, at<void>(ws, L.q), at<void>(ws, L.ks), at<void>(ws, L.vs), S, srow, rope,
             Hq, Hkv, D, rope_rows};
  launch_qkv(ctx->dt, qa, L.pa.qkv, s);
  AttnArgs ap{at<void>(ws, L.q_p), P_cap, 0, kp, vp, P_cap, nullptr, nullptr, S, prefix_lens, B, Hq, Hkv, D,
              L.n_chunks_p, L.chunk_keys_p, at<void>(ws, L.o_p),
              L.n_chunks_p > 1 ? at<void>(ws, L.apart_p) : nullptr};
  launch_attention(ctx->dt, ap, s);
  AttnArgs as{at<void>(ws, L.q), S, 1, kp, vp, P_cap, at<void>(ws, L.ks), at<void>(ws, L.vs), S, prefix_lens, B, Hq,
              Hkv, D, L.n_chunks, L.chunk_keys, at<void>(ws, L.o), L.n_chunks > 1 ? at<void>(ws, L.apart) : nullptr};
  launch_attention(ctx->dt, as, s);
  enqueue_finish(ctx, L, ws, L.pv, ev, hp, at<void>(ws, L.o_p), at<void>(ws, L.act_p), Mp, c.vlm_ffn, prow, nullptr,
                 s);
  enqueue_finish(ctx, L, ws, L.pa, ea, hs, at<void>(ws, L.o), at<void>(ws, L.act), Ms, c.act_ffn, srow, nullptr, s);
  HIP_TRY(hipGetLastError());
  return DM_OK;
}

dm_status dm_prefill_kv(dm_ctx *ctx, const dm_expert_weights *vlm, const float *prefix_embeds,
                        const int32_t *prefix_lens, int B, int P_cap, void *k_cache, void *v_cache, void *ws,
                        size_t ws_bytes, void *stream) {
  TRY(check_common(ctx, prefix_lens, B, P_cap, ws, ws_bytes, DM_OP_PREFILL));
  const dm_config &c = ctx->cfg;
  const bool fp8 = c.vlm_mlp_dtype == DM_FP8_E4M3;
  TRY(check_expert(vlm, fp8, "VLM"));
  REQUIRE(prefix_embeds && k_cache && v_cache, DM_ERR_INVALID_ARG, "prefix_embeds / k_cache / v_cache is NULL");
  REQUIRE(aligned16(prefix_embeds) && aligned16(k_cache) && aligned16(v_cache), DM_ERR_INVALID_ARG,
          "prefix_embeds and caches must be 16-byte aligned");
  TRY(set_device(ctx));
  hipStream_t s = (hipStream_t)stream;
  const Layout L = make_layout(c, ctx->es, DM_OP_PREFILL, B, P_cap);
  const int D = c.head_dim, Hkv = c.n_kv_heads, Hq = c.n_q_heads, Hv = c.vlm_hidden;
  const int Mp = B * P_cap;
  float2 *rope = at<float2>(ws, L.rope);
  const Hidden hp{at<float>(ws, L.hp), at<void>(ws, L.hg_p), at<float>(ws, L.ssq_p), Hv};
  const RowMap prow{P_cap, prefix_lens, 1, P_cap};
  const size_t layer_cache = (size_t)B * Hkv * P_cap * D;

  launch_rope_table(rope, P_cap, D, c.rope_base, s);
  launch_norm_prep(ctx->dt, prefix_embeds, hp, vlm->attn_norm, Mp, s);
  for (int l = 0; l < c.n_layers; ++l) {
    const Expert e = expert_layer(c, *vlm, l, Hv, c.vlm_ffn, ctx->es, fp8);
    void *kc = (void *)layer_ptr(k_cache, layer_cache, l, ctx->es);
    void *vc = (void *)layer_ptr(v_cache, layer_cache, l, ctx->es);
    QkvArgs qv{hp, Mp, c.rms_eps, e.w_qkv, at<void>(ws, L.q_p), kc, vc, P_cap, prow, rope, Hq, Hkv, D};
    launch_qkv(ctx->dt, qv, L.pv.qkv, s);
    if (l == c.n_layers - 1) break;  // the last layer's outputs past its K/V are never read
    AttnArgs ap{at<void>(ws, L.q_p), P_cap, 0, kc, vc, P_cap, nullptr, nullptr, c.chunk, prefix_lens, B, Hq, Hkv, D,
                L.n_chunks_p, L.chunk_keys_p, at<void>(ws, L.o_p),
                L.n_chunks_p > 1 ? at<void>(ws, L.apart_p) : nullptr};
    launch_attention(ctx->dt, ap, s);
    (fp8 ? enqueue_finish_fp8 : enqueue_finish)(ctx, L, ws, L.pv, e, hp, at<void>(ws, L.o_p), at<void>(ws, L.act_p),
                                                Mp, c.vlm_ffn, prow, vlm->attn_norm + (size_t)(l + 1) * Hv, s);
  }
  HIP_TRY(hipGetLastError());
  return DM_OK;
}

dm_status dm_quantize_fp8_rows(const void *src, uint8_t *dst, float *scales, int rows, int cols, void *stream) {
  REQUIRE(src && dst && scales, DM_ERR_INVALID_ARG, "src / dst / scales is NULL");
  REQUIRE(rows >= 1 && cols >= 1, DM_ERR_SHAPE, "rows and cols must be positive");
  REQUIRE(aligned16(src) && aligned16(dst), DM_ERR_INVALID_ARG, "src and dst must be 16-byte aligned");
  launch_fp8_quantize_rows(src, dst, scales, rows, cols, (hipStream_t)stream);
  HIP_TRY(hipGetLastError());
  return DM_OK;
}

}  // extern "C"

// C ABI of libdm: argument validation, workspace layout, and the launch sequences of the three
// operations (prefix encoding, one merged layer, suffix denoising) plus hipGraph plans.
// What each call computes is documented with its declaration in include/dm.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <mutex>
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
  size_t es;         // bytes per element of the weight dtype
  bool single_ok;    // the device holds all workgroups of the single-launch batch-1 denoise
  hipError_t scratch_status;  // result of looking up the static scratch buffer on `device`
  // dm_merged_layer and dm_train_merged_layer run independent parts of their work on a second
  // stream (forked and joined through these events); created on `device` at default priority
  static constexpr int kEvents = 8;
  hipStream_t side = nullptr;
  hipEvent_t ev[kEvents] = {};
};

// ---------------------------------------------------------------- static scratch buffer
// The workspace of dm_suffix_denoise_noalloc: a file-scope device array that every GPU the
// library runs on holds until the process ends.  In host code `scratch` names a host-side
// shadow, not device memory; its address on each device is looked up once (dm_ctx_create, with
// that device current) and only that address is handed to kernels.
namespace {
constexpr size_t kScratchBytes = DM_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Looks up this device's copy of `scratch`; the caller has made `device` current.
hipError_t scratch_setup(int device) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  if (g_scratch_ptr[device]) return hipSuccess;
  void *p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e == hipSuccess) g_scratch_ptr[device] = p;
  return e;
}

void *scratch_ptr(int device) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return device >= 0 && device < kMaxDevices ? g_scratch_ptr[device] : nullptr;
}
}  // namespace

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
  Region split_a;  // merged layer: the action expert's K-split partials (its kernels run beside the VLM's)
  Region hp, hg_p, ssq_p, q_p, kp, vp, o_p, act_p, apart_p;    // prefix side (hp: prefill only)
  Region q8_p, qs_p;                                           // FP8 MLP operand codes and row scales
  Region single;                                               // single-launch batch-1 denoise
  Region tm_tau, tm_z, tm_c, tm_mod, tm_fmod;                  // time-modulation tables of a chunk
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
constexpr int kSkinnyMaxRows = 128;  // the skinny kernel over several row blocks up to this many rows

GemmPlan plan_gemm(Dt dt, int M, int N, int K, bool split_ok) {
  GemmPlan p{};
  p.sk.k_split = 1;
  p.skinny = 0;
  p.nt = 0;  // the tiled kernel
  if (M > kSkinnyMaxRows) {
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
    // a few hundred rows (batches of 3 to 8): 128-row tiles leave most CUs idle; 64 x 128 tiles
    // make twice the workgroups, each streaming three quarters of the bytes
    const long wg = (long)(N / p.nt) * mt * p.sk.k_split;
    if (wg < 160) {
      GemmPlan q = p;
      q.bm = 64;
      q.nt = 128;
      q.sk.k_split = 1;
      const int mt64 = (M + 63) / 64;
      if (split_ok)
        while ((N / 128) * mt64 * q.sk.k_split < 200 && q.sk.k_split < 8 && K % (2 * q.sk.k_split * 64) == 0 &&
               K / (2 * q.sk.k_split) >= 256)
          q.sk.k_split *= 2;
      const long wg64 = (long)(N / 128) * mt64 * q.sk.k_split;
      if (wg64 > wg && wg64 <= 256) return q;
    }
    return p;
  }
  // Up to 64 rows one row block; more rows (small batches above one sample) take several row
  // blocks of 16 * rt rows (grid.z), each workgroup re-reading its weight slice, which the
  // workgroups of one column slice (same XCD) find in L2.
  const int kq = gemm_k_quantum(dt);  // K per k-chunk across the 4 waves
  auto blocks = [&](int rows) { return (M + rows - 1) / rows; };
  if (split_ok && N % 16 == 0 && K % (4 * kq) == 0 && K / (4 * kq) <= 8 && (N / 16) * blocks(16) >= 128) {
    // residual projections: 16 waves per workgroup cover the whole K of 16 columns x 16 (or 32)
    // rows, enough workgroups without a K split, so the residual epilogue runs in the same
    // launch (batch 1, O: 7.7 -> 6.7 us in isolation, one launch fewer)
    p.skinny = 1;
    p.nt = 16;
    p.rt = (N / 16) * blocks(16) <= 256 ? 1 : 2;
    p.nw = 16;
    return p;
  }
  const int nt = N % 32 == 0 ? 32 : 16;
  int ks = 1;
  if (split_ok) {
    while ((N / nt) * ks * blocks(64) < 256 && ks < 16 && K % (2 * ks * kq) == 0) ks *= 2;
    while (K / (ks * kq) > 8 && ks < 16 && K % (2 * ks * kq) == 0) ks *= 2;
  }
  if (K % (ks * kq) != 0 || K / (ks * kq) > 8) return p;
  p.skinny = 1;
  p.nt = nt;
  p.sk.k_split = ks;
  // half-height workgroups when twice as many still fit the 256 CUs in one round: each reads
  // half the activation rows, and twice the CUs pull the weights (QKV at batch 1: 9.2 -> 7.5 us)
  if (M > 32 && (size_t)(N / nt) * ks * blocks(32) <= 256) p.rt = 2;
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

// The batch-1 denoise runs as one launch per chunk (persist.hip) for the DM0-base action expert
// shapes, unless the config asks for the multi-kernel sequence.
bool single_launch_shape(const dm_config &c, int B, int P_cap) {
  return !(c.flags & (DM_FLAG_MULTI_KERNEL | DM_FLAG_TIME_MODULATION | DM_FLAG_QK_NORM)) &&
         persist_supported(c.n_layers, c.act_hidden, c.act_ffn, c.n_q_heads, c.n_kv_heads, c.head_dim, c.chunk, c.action_dim, B,
                           P_cap, c.dtype == DM_BF16);
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
    if (op == DM_OP_MERGED_LAYER) {  // a region of its own: the two experts' finishes overlap
      if (split) L.put(L.split_a, split);
      split = 0;
    }
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
    if (op == DM_OP_DENOISE && single_launch_shape(c, B, P_cap)) L.put(L.single, persist_ws_bytes(S, c.action_dim));
    if (op == DM_OP_DENOISE && (c.flags & DM_FLAG_TIME_MODULATION)) {
      const size_t rows = DM_TMOD_MAX_STEPS;
      L.put(L.tm_tau, rows * Ha * sizeof(float));
      L.put(L.tm_z, rows * Ha * sizeof(float));
      L.put(L.tm_c, rows * Ha * sizeof(float));
      L.put(L.tm_mod, rows * c.n_layers * 6 * Ha * sizeof(float));
      L.put(L.tm_fmod, rows * 2 * Ha * sizeof(float));
    }
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

constexpr size_t kTrainSplitFloats = (size_t)24 << 20;

// fp32 buffers of one training step (dm_train_merged_layer): M = B*S action rows, Mp = B*P_cap
// prefix rows, T = P_cap + S joined keys.
struct TrainLayout {
  Region x, u, v, dv, h0, n1, r1, qkv, dqkv, K, V, dK, dV, sc, dp, o, dO, h1, n2, r2, gt, up, act, dgt, dup, dact, h2,
      nf, rf, dnf, dh2, dn2, dh1, dn1, dh0, np, rp, kvp, dkvp, dnp, split, cpart, split2, cpart2;
  size_t total = 0;
  void put(Region &r, size_t floats) {
    r.off = total;
    r.bytes = floats * sizeof(float);
    total += up256(r.bytes);
  }
};

TrainLayout train_layout(const dm_config &c, int B, int P_cap) {
  TrainLayout L;
  const size_t S = c.chunk, A = c.action_dim, D = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
  const size_t Ha = c.act_hidden, Hv = c.vlm_hidden, F = c.act_ffn, QKV = (Hq + 2 * Hkv) * D;
  const size_t M = (size_t)B * S, Mp = (size_t)B * P_cap, T = P_cap + S;
  for (Region *r : {&L.x, &L.u, &L.v, &L.dv}) L.put(*r, M * A);
  for (Region *r : {&L.h0, &L.n1, &L.h1, &L.n2, &L.h2, &L.nf, &L.dnf, &L.dh2, &L.dn2, &L.dh1, &L.dn1, &L.dh0})
    L.put(*r, M * Ha);
  for (Region *r : {&L.r1, &L.r2, &L.rf}) L.put(*r, M);
  for (Region *r : {&L.qkv, &L.dqkv}) L.put(*r, M * QKV);
  for (Region *r : {&L.K, &L.V, &L.dK, &L.dV}) L.put(*r, (size_t)B * Hkv * T * D);
  for (Region *r : {&L.sc, &L.dp}) L.put(*r, (size_t)B * Hq * S * T);
  for (Region *r : {&L.o, &L.dO}) L.put(*r, M * Hq * D);
  for (Region *r : {&L.gt, &L.up, &L.act, &L.dgt, &L.dup, &L.dact}) L.put(*r, M * F);
  for (Region *r : {&L.np, &L.dnp}) L.put(*r, Mp * Hv);
  L.put(L.rp, Mp);
  for (Region *r : {&L.kvp, &L.dkvp}) L.put(*r, Mp * 2 * Hkv * D);
  L.put(L.split, kTrainSplitFloats);  // split-K partial sums of the products with few tiles
  L.put(L.cpart, std::max(colsum_part_floats((int)M, (int)std::max(Ha, A)), colsum_part_floats((int)Mp, (int)Hv)));
  // the same two for the products and column sums on the side stream
  L.put(L.split2, kTrainSplitFloats);
  L.put(L.cpart2, colsum_part_floats((int)Mp, (int)Hv));
  return L;
}

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
  REQUIRE((c->flags & ~(DM_FLAG_MULTI_KERNEL | DM_FLAG_TIME_MODULATION | DM_FLAG_QK_NORM)) == 0, DM_ERR_INVALID_ARG,
          "unknown flags 0x%x", c->flags);
  REQUIRE(!(c->flags & DM_FLAG_TIME_MODULATION) || c->act_hidden <= 1024, DM_ERR_UNSUPPORTED,
          "the time-modulated action expert supports act_hidden <= 1024");
  return DM_OK;
}

dm_status check_expert(const dm_expert_weights *w, bool fp8, const char *name, bool qk) {
  REQUIRE(w, DM_ERR_INVALID_ARG, "%s weights are NULL", name);
  REQUIRE(qk == (w->q_norm != nullptr) && qk == (w->k_norm != nullptr), DM_ERR_INVALID_ARG,
          qk ? "%s weights: DM_FLAG_QK_NORM needs q_norm and k_norm" : "%s weights: q_norm / k_norm without DM_FLAG_QK_NORM",
          name);
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
  const float *q_norm = nullptr, *k_norm = nullptr;                   // QK-norm only
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
  if (c.flags & DM_FLAG_QK_NORM) {
    e.q_norm = w.q_norm + (size_t)l * c.head_dim;
    e.k_norm = w.k_norm + (size_t)l * c.head_dim;
  }
  return e;
}

SplitK splitk(const Layout &L, void *ws, const GemmPlan &p) {
  SplitK s = p.sk;
  s.part = L.split.bytes ? at<float>(ws, L.split) : nullptr;
  return s;
}

// One expert's O-projection + residual (enqueue_oproj), then its MLP + residual (enqueue_mlp).
// `next_attn_norm` is the gain of the norm that follows the layer (NULL after the last layer of
// a stack).
void enqueue_oproj(const dm_ctx *ctx, const Layout &L, void *ws, const ExpertPlans &pl, const Expert &e,
                   const Hidden &hid, const void *o, int M, RowMap rows, hipStream_t s) {
  const dm_config &c = ctx->cfg;
  GemmPlan po = pl.o;
  po.sk = splitk(L, ws, pl.o);
  ResidArgs ro{o, M, c.n_q_heads * c.head_dim, e.w_o, hid, e.mlp_norm, rows};
  launch_resid(ctx->dt, ro, po, s);
}
void enqueue_mlp(const dm_ctx *ctx, const Layout &L, void *ws, const ExpertPlans &pl, const Expert &e,
                 const Hidden &hid, void *act, int M, int F, RowMap rows, const float *next_attn_norm,
                 hipStream_t s) {
  const dm_config &c = ctx->cfg;
  GemmPlan pg = pl.gu, pd = pl.down;
  pd.sk = splitk(L, ws, pl.down);
  SwigluArgs sg{hid, M, F, c.rms_eps, e.w_gate, e.w_up, act, rows};
  launch_swiglu(ctx->dt, sg, pg, s);
  ResidArgs rd{act, M, F, e.w_down, hid, next_attn_norm, rows};
  launch_resid(ctx->dt, rd, pd, s);
}
void enqueue_finish(const dm_ctx *ctx, const Layout &L, void *ws, const ExpertPlans &pl, const Expert &e,
                    const Hidden &hid, const void *o, void *act, int M, int F, RowMap rows,
                    const float *next_attn_norm, hipStream_t s) {
  enqueue_oproj(ctx, L, ws, pl, e, hid, o, M, rows, s);
  enqueue_mlp(ctx, L, ws, pl, e, hid, act, M, F, rows, next_attn_norm, s);
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

// The time-modulated action expert (page "DM0.5: High-Performance Embodied VLA ...", section 5.2):
// the chunk's modulation tables first (time MLP and every layer's modulator for all Euler steps:
// t is shared by the batch, so each modulator weight is read once per chunk), then per layer a
// modulated norm before each sublayer (its GEMM takes the normalised operand as is) and the
// residual gates in the O and down epilogues.
dm_status enqueue_denoise_tmod(const dm_ctx *ctx, const Layout &L, const dm_action_weights *aw, const void *k_cache,
                               const void *v_cache, const int32_t *lens, int B, int P_cap, float *x, int num_steps,
                               void *ws, hipStream_t s) {
  const dm_config &c = ctx->cfg;
  const dm_time_modulation &tm = *aw->tmod;
  const int S = c.chunk, Ha = c.act_hidden, Fa = c.act_ffn, D = c.head_dim, Hkv = c.n_kv_heads, NL = c.n_layers;
  const int M = B * S;
  const float eps = c.rms_eps;
  float *tau = at<float>(ws, L.tm_tau), *z = at<float>(ws, L.tm_z), *cc = at<float>(ws, L.tm_c);
  float *mod = at<float>(ws, L.tm_mod), *fmod = at<float>(ws, L.tm_fmod);
  launch_tau_table(tau, num_steps, Ha, s);
  launch_rows_gemv(DT_F32, tau, num_steps, Ha, tm.w_in, tm.b_in, z, Ha, false, s);
  launch_rows_gemv(DT_F32, z, num_steps, Ha, tm.w_out, tm.b_out, cc, Ha, true, s);
  launch_rows_gemv(ctx->dt, cc, num_steps, Ha, tm.w_mod, tm.b_mod, mod, NL * 6 * Ha, true, s);
  launch_rows_gemv(ctx->dt, cc, num_steps, Ha, tm.w_fmod, tm.b_fmod, fmod, 2 * Ha, true, s);

  float2 *rope = at<float2>(ws, L.rope);
  const Hidden hid{at<float>(ws, L.h), at<void>(ws, L.hg), at<float>(ws, L.ssq), Ha};
  const Hidden normed{hid.h, hid.hg, nullptr, Ha};  // operand already normalised: no row scale
  void *q = at<void>(ws, L.q), *ks = at<void>(ws, L.ks), *vs = at<void>(ws, L.vs);
  void *o = at<void>(ws, L.o), *act = at<void>(ws, L.act);
  const RowMap rows{S, lens, 0, P_cap};
  const size_t layer_cache = (size_t)B * Hkv * P_cap * D;
  launch_rope_table(rope, P_cap + S, D, c.rope_base, s);
  float2 *rope_rows = at<float2>(ws, L.rope_rows);
  launch_rope_rows(rope, lens, P_cap, B, S, D, rope_rows, s);
  GemmPlan po = L.pa.o, pd = L.pa.down;
  po.sk = splitk(L, ws, L.pa.o);
  pd.sk = splitk(L, ws, L.pa.down);
  for (int k = 0; k < num_steps; ++k) {
    const float t = 1.0f - (float)k / (float)num_steps;
    launch_embed(ctx->dt, x, aw->w_in, aw->b_in, hid, nullptr, M, c.action_dim, t, s);
    for (int l = 0; l < NL; ++l) {
      const float *m = mod + ((size_t)k * NL + l) * 6 * Ha;  // attention scale, shift, gate; MLP scale, shift, gate
      const Expert e = expert_layer(c, aw->body, l, Ha, Fa, ctx->es);
      launch_mod_norm(ctx->dt, hid.h, hid.hg, m, m + Ha, M, Ha, eps, s);
      QkvArgs qa{normed, M, eps, e.w_qkv, q, ks, vs, S, rows, rope, c.n_q_heads, Hkv, D, rope_rows, e.q_norm, e.k_norm};
      launch_qkv(ctx->dt, qa, L.pa.qkv, s);
      AttnArgs aa{q, S, 1,
                  layer_ptr(k_cache, layer_cache, l, ctx->es), layer_ptr(v_cache, layer_cache, l, ctx->es), P_cap,
                  ks, vs, S, lens, B, c.n_q_heads, Hkv, D, L.n_chunks, L.chunk_keys, o,
                  L.n_chunks > 1 ? at<void>(ws, L.apart) : nullptr};
      launch_attention(ctx->dt, aa, s);
      ResidArgs ro{o, M, c.n_q_heads * D, e.w_o, hid, nullptr, rows};
      ro.gate = m + 2 * Ha;
      launch_resid(ctx->dt, ro, po, s);
      launch_mod_norm(ctx->dt, hid.h, hid.hg, m + 3 * Ha, m + 4 * Ha, M, Ha, eps, s);
      SwigluArgs sg{normed, M, Fa, eps, e.w_gate, e.w_up, act, rows};
      launch_swiglu(ctx->dt, sg, L.pa.gu, s);
      ResidArgs rd{act, M, Fa, e.w_down, hid, nullptr, rows};
      rd.gate = m + 5 * Ha;
      launch_resid(ctx->dt, rd, pd, s);
    }
    const float *f = fmod + (size_t)k * 2 * Ha;
    launch_velocity_euler(hid.h, nullptr, aw->w_out, aw->b_out, x, M, Ha, c.action_dim, eps, num_steps, s, f, f + Ha);
  }
  return DM_OK;
}

dm_status enqueue_denoise(const dm_ctx *ctx, const dm_action_weights *aw, const void *k_cache, const void *v_cache,
                          const int32_t *lens, int B, int P_cap, float *x, int num_steps, void *ws, hipStream_t s) {
  const dm_config &c = ctx->cfg;
  const Layout L = make_layout(c, ctx->es, DM_OP_DENOISE, B, P_cap);
  if (c.flags & DM_FLAG_TIME_MODULATION)
    return enqueue_denoise_tmod(ctx, L, aw, k_cache, v_cache, lens, B, P_cap, x, num_steps, ws, s);
  if (ctx->single_ok && L.single.bytes) {
    const dm_expert_weights &w = aw->body;
    PersistLaunch p{w.w_qkv, w.w_o, w.w_gate, w.w_up, w.w_down, w.attn_norm, w.mlp_norm, aw->w_in, aw->b_in,
                    aw->final_norm, aw->w_out, aw->b_out, k_cache, v_cache, lens, x, c.n_layers, c.chunk,
                    c.action_dim, P_cap, num_steps, c.rms_eps, c.rope_base, at<void>(ws, L.single)};
    HIP_TRY(launch_denoise_persistent(p, s));
    return DM_OK;
  }
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
      QkvArgs qa{hid, M, c.rms_eps, e.w_qkv, q, ks, vs, S, rows, rope, c.n_q_heads, Hkv, D, rope_rows, e.q_norm, e.k_norm};
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
  TRY(check_expert(&aw->body, false, "action", (ctx->cfg.flags & DM_FLAG_QK_NORM) != 0));
  const void *ptrs[] = {aw->w_in, aw->b_in, aw->final_norm, aw->w_out, aw->b_out};
  for (const void *p : ptrs) {
    REQUIRE(p, DM_ERR_INVALID_ARG, "action head: a tensor pointer is NULL");
    REQUIRE(aligned16(p), DM_ERR_INVALID_ARG, "action head: a tensor pointer is not 16-byte aligned");
  }
  const bool tmod = (ctx->cfg.flags & DM_FLAG_TIME_MODULATION) != 0;
  REQUIRE(tmod == (aw->tmod != nullptr), DM_ERR_INVALID_ARG,
          tmod ? "DM_FLAG_TIME_MODULATION needs action weights with tmod set"
               : "action weights carry tmod but the config has no DM_FLAG_TIME_MODULATION");
  if (tmod) {
    const dm_time_modulation &t = *aw->tmod;
    const void *tp[] = {t.w_in, t.b_in, t.w_out, t.b_out, t.w_mod, t.b_mod, t.w_fmod, t.b_fmod};
    for (const void *p : tp) {
      REQUIRE(p, DM_ERR_INVALID_ARG, "time modulation: a tensor pointer is NULL");
      REQUIRE(aligned16(p), DM_ERR_INVALID_ARG, "time modulation: a tensor pointer is not 16-byte aligned");
    }
  }
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
  REQUIRE(!(ctx->cfg.flags & DM_FLAG_TIME_MODULATION) || num_steps <= DM_TMOD_MAX_STEPS, DM_ERR_UNSUPPORTED,
          "the time-modulated expert supports at most %d Euler steps (got %d)", DM_TMOD_MAX_STEPS, num_steps);
  return DM_OK;
}

dm_status check_prefill(dm_ctx *ctx, const dm_expert_weights *vlm, const float *prefix_embeds, const int32_t *lens,
                        int B, int P_cap, void *k_cache, void *v_cache, void *ws, size_t ws_bytes) {
  TRY(check_common(ctx, lens, B, P_cap, ws, ws_bytes, DM_OP_PREFILL));
  const dm_config &c = ctx->cfg;
  TRY(check_expert(vlm, c.vlm_mlp_dtype == DM_FP8_E4M3, "VLM", (c.flags & DM_FLAG_QK_NORM) != 0));
  REQUIRE(prefix_embeds && k_cache && v_cache, DM_ERR_INVALID_ARG, "prefix_embeds / k_cache / v_cache is NULL");
  REQUIRE(aligned16(prefix_embeds) && aligned16(k_cache) && aligned16(v_cache), DM_ERR_INVALID_ARG,
          "prefix_embeds and caches must be 16-byte aligned");
  return DM_OK;
}

// The prefix encoding's launches on `s` (arguments already checked).
void enqueue_prefill(const dm_ctx *ctx, const dm_expert_weights *vlm, const float *prefix_embeds,
                     const int32_t *prefix_lens, int B, int P_cap, void *k_cache, void *v_cache, void *ws,
                     hipStream_t s) {
  const dm_config &c = ctx->cfg;
  const bool fp8 = c.vlm_mlp_dtype == DM_FP8_E4M3;
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
    QkvArgs qv{hp, Mp, c.rms_eps, e.w_qkv, at<void>(ws, L.q_p), kc, vc, P_cap, prow, rope, Hq, Hkv, D, nullptr,
               e.q_norm, e.k_norm};
    launch_qkv(ctx->dt, qv, L.pv.qkv, s);
    if (l == c.n_layers - 1) break;  // the last layer's outputs past its K/V are never read
    AttnArgs ap{at<void>(ws, L.q_p), P_cap, 0, kc, vc, P_cap, nullptr, nullptr, c.chunk, prefix_lens, B, Hq, Hkv, D,
                L.n_chunks_p, L.chunk_keys_p, at<void>(ws, L.o_p),
                L.n_chunks_p > 1 ? at<void>(ws, L.apart_p) : nullptr};
    launch_attention(ctx->dt, ap, s);
    (fp8 ? enqueue_finish_fp8 : enqueue_finish)(ctx, L, ws, L.pv, e, hp, at<void>(ws, L.o_p), at<void>(ws, L.act_p),
                                                Mp, c.vlm_ffn, prow, vlm->attn_norm + (size_t)(l + 1) * Hv, s);
  }
}

dm_status set_device(const dm_ctx *ctx) {
  int cur = -1;
  HIP_TRY(hipGetDevice(&cur));
  if (cur != ctx->device) HIP_TRY(hipSetDevice(ctx->device));
  return DM_OK;
}

// Captures what `enqueue(capture_stream)` launches into a graph on a private stream, then
// instantiates it and uploads it on `stream` (which is synchronised).  On failure nothing is
// kept and the enqueue's own status, or DM_ERR_HIP, is returned.
template <class F>
dm_status capture_graph(hipStream_t stream, F &&enqueue, hipGraph_t *graph_out, hipGraphExec_t *exec_out) {
  hipStream_t cs = nullptr;
  HIP_TRY(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking));
  hipGraph_t graph = nullptr;
  hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeRelaxed);
  if (e != hipSuccess) {
    (void)hipStreamDestroy(cs);
    return fail(DM_ERR_HIP, "hipStreamBeginCapture: %s", hipGetErrorString(e));
  }
  const dm_status st = enqueue(cs);
  const hipError_t le = hipGetLastError();
  e = hipStreamEndCapture(cs, &graph);
  (void)hipStreamDestroy(cs);
  if (st != DM_OK || le != hipSuccess || e != hipSuccess) {
    if (graph) (void)hipGraphDestroy(graph);
    if (st != DM_OK) return st;
    return fail(DM_ERR_HIP, "graph capture: %s", hipGetErrorString(le != hipSuccess ? le : e));
  }
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return fail(DM_ERR_HIP, "hipGraphInstantiate: %s", hipGetErrorString(e));
  }
  e = hipGraphUpload(exec, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    return fail(DM_ERR_HIP, "hipGraphUpload: %s", hipGetErrorString(e));
  }
  *graph_out = graph;
  *exec_out = exec;
  return DM_OK;
}

}  // namespace

// A fixed-contract engine: one device allocation holding the static buffers, and the captured
// graph of the prefix encoding followed by the denoise over them.
struct dm_engine {
  int device;
  dm_engine_contract contract;
  void *mem;
  float *embeds;
  int32_t *lens;
  float *x;
  size_t embeds_bytes, x_bytes;
  hipGraph_t graph;
  hipGraphExec_t exec;
};

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
  // the single-launch denoise needs all of its workgroups resident at once
  // and, once per device, the address of the static scratch buffer
  int prev = -1;
  ctx->single_ok = false;
  ctx->scratch_status = hipErrorNotReady;
  if (hipGetDevice(&prev) == hipSuccess && hipSetDevice(device) == hipSuccess) {
    ctx->single_ok = persist_check_device(device) == hipSuccess;
    ctx->scratch_status = scratch_setup(device);
    hipError_t e = hipStreamCreateWithFlags(&ctx->side, hipStreamNonBlocking);
    for (int k = 0; k < dm_ctx::kEvents && e == hipSuccess; ++k)
      e = hipEventCreateWithFlags(&ctx->ev[k], hipEventDisableTiming);
    (void)hipSetDevice(prev);
    if (e != hipSuccess) {
      dm_ctx_destroy(ctx);
      (void)hipGetLastError();
      return fail(DM_ERR_HIP, "creating the context's side stream / events: %s", hipGetErrorString(e));
    }
  }
  (void)hipGetLastError();
  *out = ctx;
  return DM_OK;
}

void dm_ctx_destroy(dm_ctx *ctx) {
  if (!ctx) return;
  int cur = -1;
  const bool back = hipGetDevice(&cur) == hipSuccess && cur != ctx->device && hipSetDevice(ctx->device) == hipSuccess;
  for (hipEvent_t e : ctx->ev)
    if (e) (void)hipEventDestroy(e);
  if (ctx->side) (void)hipStreamDestroy(ctx->side);
  if (back) (void)hipSetDevice(cur);
  (void)hipGetLastError();
  delete ctx;
}

size_t dm_workspace_bytes(const dm_ctx *ctx, dm_op op, int B, int P_cap) {
  if (!ctx || B < 1 || P_cap < 1) return 0;
  if (op == DM_OP_TRAIN) return train_layout(ctx->cfg, B, P_cap).total;
  if (op != DM_OP_PREFILL && op != DM_OP_MERGED_LAYER && op != DM_OP_DENOISE) return 0;
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

dm_status dm_suffix_denoise_noalloc(dm_ctx *ctx, const dm_action_weights *aw, const void *k_cache,
                                    const void *v_cache, const int32_t *prefix_lens, int B, int P_cap, float *x,
                                    int num_steps, void *stream) {
  REQUIRE(ctx, DM_ERR_INVALID_ARG, "ctx is NULL");
  REQUIRE(B >= 1 && P_cap >= 1, DM_ERR_INVALID_ARG, "B and P_cap must be >= 1");
  const size_t need = make_layout(ctx->cfg, ctx->es, DM_OP_DENOISE, B, P_cap).total;
  REQUIRE(need <= kScratchBytes, DM_ERR_WORKSPACE,
          "dm_suffix_denoise_noalloc: B=%d, P_cap=%d need %zu bytes of scratch, more than the static %zu-byte "
          "buffer; use dm_suffix_denoise with a workspace",
          B, P_cap, need, kScratchBytes);
  void *ws = scratch_ptr(ctx->device);
  REQUIRE(ws, DM_ERR_HIP, "no address of the static scratch buffer on device %d: %s", ctx->device,
          hipGetErrorString(ctx->scratch_status));
  TRY(check_denoise(ctx, aw, k_cache, v_cache, prefix_lens, B, P_cap, x, num_steps, ws, kScratchBytes));
  TRY(set_device(ctx));
  TRY(enqueue_denoise(ctx, aw, k_cache, v_cache, prefix_lens, B, P_cap, x, num_steps, ws, (hipStream_t)stream));
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
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  TRY(capture_graph(
      (hipStream_t)stream,
      [&](hipStream_t cs) { return enqueue_denoise(ctx, aw, k_cache, v_cache, prefix_lens, B, P_cap, x, num_steps, ws, cs); },
      &graph, &exec));
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
  int cur = -1;
  HIP_TRY(hipGetDevice(&cur));
  if (cur != plan->device) HIP_TRY(hipSetDevice(plan->device));
  HIP_TRY(hipGraphLaunch(plan->exec, (hipStream_t)stream));
  return DM_OK;
}

void dm_denoise_plan_destroy(dm_plan *plan) {
  if (!plan) return;
  (void)hipGraphExecDestroy(plan->exec);
  (void)hipGraphDestroy(plan->graph);
  delete plan;
}

dm_status dm_engine_create(dm_ctx *ctx, const dm_expert_weights *vlm, const dm_action_weights *aw, int B, int P_cap,
                           int num_steps, void *stream, dm_engine **out) {
  REQUIRE(out, DM_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  REQUIRE(ctx, DM_ERR_INVALID_ARG, "ctx is NULL");
  REQUIRE(B >= 1 && B <= 4096, DM_ERR_SHAPE, "B must be 1..4096 (got %d)", B);
  REQUIRE(P_cap >= 1 && P_cap <= 65536, DM_ERR_SHAPE, "P_cap must be 1..65536 (got %d)", P_cap);
  REQUIRE(num_steps >= 1 && num_steps <= 1000, DM_ERR_SHAPE, "num_steps must be 1..1000 (got %d)", num_steps);
  const dm_config &c = ctx->cfg;
  TRY(check_expert(vlm, c.vlm_mlp_dtype == DM_FP8_E4M3, "VLM", (c.flags & DM_FLAG_QK_NORM) != 0));
  TRY(check_action(ctx, aw));
  REQUIRE(!(c.flags & DM_FLAG_TIME_MODULATION) || num_steps <= DM_TMOD_MAX_STEPS, DM_ERR_UNSUPPORTED,
          "the time-modulated expert supports at most %d Euler steps (got %d)", DM_TMOD_MAX_STEPS, num_steps);
  // one allocation: embeddings, lengths, x, K cache, V cache, workspace (each 256-byte aligned)
  const size_t embeds_bytes = (size_t)B * P_cap * c.vlm_hidden * sizeof(float);
  const size_t lens_bytes = (size_t)B * sizeof(int32_t);
  const size_t x_bytes = (size_t)B * c.chunk * c.action_dim * sizeof(float);
  const size_t cache_bytes = (size_t)c.n_layers * B * c.n_kv_heads * P_cap * c.head_dim * ctx->es;
  const size_t ws_bytes = std::max(make_layout(c, ctx->es, DM_OP_PREFILL, B, P_cap).total,
                                   make_layout(c, ctx->es, DM_OP_DENOISE, B, P_cap).total);
  const size_t o_lens = up256(embeds_bytes), o_x = o_lens + up256(lens_bytes), o_k = o_x + up256(x_bytes);
  const size_t o_v = o_k + up256(cache_bytes), o_ws = o_v + up256(cache_bytes), total = o_ws + up256(ws_bytes);
  TRY(set_device(ctx));
  hipStream_t s = (hipStream_t)stream;
  void *mem = nullptr;
  HIP_TRY(hipMalloc(&mem, total));
  char *base = (char *)mem;
  float *embeds = (float *)base;
  int32_t *lens = (int32_t *)(base + o_lens);
  float *x = (float *)(base + o_x);
  void *kc = base + o_k, *vc = base + o_v, *ws = base + o_ws;
  hipError_t e = hipMemsetAsync(mem, 0, total, s);  // before capture, never inside the graph
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    (void)hipFree(mem);
    return fail(DM_ERR_HIP, "clearing the engine buffers: %s", hipGetErrorString(e));
  }
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  const dm_status st = capture_graph(
      s,
      [&](hipStream_t cs) {
        enqueue_prefill(ctx, vlm, embeds, lens, B, P_cap, kc, vc, ws, cs);
        return enqueue_denoise(ctx, aw, kc, vc, lens, B, P_cap, x, num_steps, ws, cs);
      },
      &graph, &exec);
  if (st != DM_OK) {
    (void)hipFree(mem);
    return st;
  }
  dm_engine *eng = new (std::nothrow) dm_engine;
  if (!eng) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    (void)hipFree(mem);
    return fail(DM_ERR_INVALID_ARG, "out of host memory");
  }
  eng->device = ctx->device;
  eng->contract = dm_engine_contract{B, P_cap, num_steps, c.chunk, c.action_dim, c.vlm_hidden};
  eng->mem = mem;
  eng->embeds = embeds;
  eng->lens = lens;
  eng->x = x;
  eng->embeds_bytes = embeds_bytes;
  eng->x_bytes = x_bytes;
  eng->graph = graph;
  eng->exec = exec;
  *out = eng;
  return DM_OK;
}

dm_status dm_engine_contract_get(const dm_engine *eng, dm_engine_contract *out) {
  REQUIRE(eng && out, DM_ERR_INVALID_ARG, "engine / out is NULL");
  *out = eng->contract;
  return DM_OK;
}

dm_status dm_engine_run(dm_engine *eng, const dm_engine_request *req, void *stream) {
  REQUIRE(eng && req, DM_ERR_INVALID_ARG, "engine / request is NULL");
  const dm_engine_contract &k = eng->contract;
  REQUIRE(req->batch == k.batch && req->prefix_cap == k.prefix_cap && req->num_steps == k.num_steps,
          DM_ERR_PLAN_MISMATCH,
          "request (batch %d, prefix_cap %d, num_steps %d) differs from the engine's contract (batch %d, prefix_cap "
          "%d, num_steps %d)",
          req->batch, req->prefix_cap, req->num_steps, k.batch, k.prefix_cap, k.num_steps);
  REQUIRE(req->prefix_embeds && req->prefix_lens && req->noise && req->actions, DM_ERR_INVALID_ARG,
          "a request buffer is NULL");
  for (int b = 0; b < k.batch; ++b)
    REQUIRE(req->prefix_lens[b] >= 0 && req->prefix_lens[b] <= k.prefix_cap, DM_ERR_SHAPE,
            "prefix_lens[%d] = %d lies outside 0..%d", b, req->prefix_lens[b], k.prefix_cap);
  int cur = -1;
  HIP_TRY(hipGetDevice(&cur));
  if (cur != eng->device) HIP_TRY(hipSetDevice(eng->device));
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(hipMemcpyAsync(eng->embeds, req->prefix_embeds, eng->embeds_bytes, hipMemcpyHostToDevice, s));
  HIP_TRY(hipMemcpyAsync(eng->lens, req->prefix_lens, (size_t)k.batch * sizeof(int32_t), hipMemcpyHostToDevice, s));
  HIP_TRY(hipMemcpyAsync(eng->x, req->noise, eng->x_bytes, hipMemcpyHostToDevice, s));
  HIP_TRY(hipGraphLaunch(eng->exec, s));
  HIP_TRY(hipMemcpyAsync(req->actions, eng->x, eng->x_bytes, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  return DM_OK;
}

dm_status dm_engine_replay(dm_engine *eng, void *stream) {
  REQUIRE(eng, DM_ERR_INVALID_ARG, "engine is NULL");
  int cur = -1;
  HIP_TRY(hipGetDevice(&cur));
  if (cur != eng->device) HIP_TRY(hipSetDevice(eng->device));
  HIP_TRY(hipGraphLaunch(eng->exec, (hipStream_t)stream));
  return DM_OK;
}

dm_status dm_engine_buffers(const dm_engine *eng, float **prefix_embeds, int32_t **prefix_lens, float **x) {
  REQUIRE(eng, DM_ERR_INVALID_ARG, "engine is NULL");
  if (prefix_embeds) *prefix_embeds = eng->embeds;
  if (prefix_lens) *prefix_lens = eng->lens;
  if (x) *x = eng->x;
  return DM_OK;
}

void dm_engine_destroy(dm_engine *eng) {
  if (!eng) return;
  int cur = -1;
  const bool back = hipGetDevice(&cur) == hipSuccess && cur != eng->device && hipSetDevice(eng->device) == hipSuccess;
  (void)hipGraphExecDestroy(eng->exec);
  (void)hipGraphDestroy(eng->graph);
  (void)hipFree(eng->mem);
  if (back) (void)hipSetDevice(cur);
  delete eng;
}

dm_status dm_merged_layer(dm_ctx *ctx, const dm_expert_weights *vlm, const dm_expert_weights *act, int layer,
                          float *h_prefix, float *h_suffix, const int32_t *prefix_lens, int B, int P_cap, void *k_out,
                          void *v_out, void *ws, size_t ws_bytes, void *stream) {
  TRY(check_common(ctx, prefix_lens, B, P_cap, ws, ws_bytes, DM_OP_MERGED_LAYER));
  const dm_config &c = ctx->cfg;
  REQUIRE(c.vlm_mlp_dtype == c.dtype, DM_ERR_UNSUPPORTED, "dm_merged_layer runs the VLM MLP in the weight dtype");
  REQUIRE(!(c.flags & DM_FLAG_TIME_MODULATION), DM_ERR_UNSUPPORTED,
          "the time-modulated action expert needs the flow time: only dm_suffix_denoise runs it");
  TRY(check_expert(vlm, false, "VLM", (c.flags & DM_FLAG_QK_NORM) != 0));
  TRY(check_expert(act, false, "action", (c.flags & DM_FLAG_QK_NORM) != 0));
  REQUIRE(layer >= 0 && layer < c.n_layers, DM_ERR_SHAPE, "layer %d out of range", layer);
  REQUIRE(h_prefix && h_suffix, DM_ERR_INVALID_ARG, "h_prefix / h_suffix is NULL");
  REQUIRE(aligned16(h_prefix) && aligned16(h_suffix), DM_ERR_INVALID_ARG, "hidden streams must be 16-byte aligned");
  REQUIRE((k_out == nullptr) == (v_out == nullptr), DM_ERR_INVALID_ARG, "k_out and v_out must both be set or NULL");
  REQUIRE(!k_out || (aligned16(k_out) && aligned16(v_out)), DM_ERR_INVALID_ARG, "k_out / v_out must be aligned");
  REQUIRE(ctx->side, DM_ERR_HIP, "the context has no side stream (dm_ctx_create could not make the device current)");
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

  // The two experts' kernels share only the prefix K/V and the RoPE table, so they run on two
  // streams: the VLM expert's on `stream`, the action expert's on the context's side stream
  // (the action rows' GEMMs are small and leave most CUs to the prefix rows' GEMMs).  The side
  // stream starts after the RoPE table, its attention waits for the prefix K/V, and `stream`
  // waits for the side stream's last kernel, so the call's work is ordered on `stream` alone.
  // Launches are issued one at a time from the host, so the order of enqueueing decides what
  // can overlap: the VLM chain (the longer one) up to its O-projection first, then the action
  // expert up to its attention (which then runs beside the VLM O-projection and MLP), the VLM MLP,
  // and the rest of the action expert.
  hipStream_t sa = ctx->side;
  launch_rope_table(rope, P_cap + S, D, c.rope_base, s);
  HIP_TRY(hipEventRecord(ctx->ev[0], s));
  launch_norm_prep(ctx->dt, h_prefix, hp, ev.attn_norm, Mp, s);
  QkvArgs qv{hp, Mp, c.rms_eps, ev.w_qkv, at<void>(ws, L.q_p), kp, vp, P_cap, prow, rope, Hq, Hkv, D, nullptr,
             ev.q_norm, ev.k_norm};
  launch_qkv(ctx->dt, qv, L.pv.qkv, s);
  HIP_TRY(hipEventRecord(ctx->ev[1], s));
  AttnArgs ap{at<void>(ws, L.q_p), P_cap, 0, kp, vp, P_cap, nullptr, nullptr, S, prefix_lens, B, Hq, Hkv, D,
              L.n_chunks_p, L.chunk_keys_p, at<void>(ws, L.o_p),
              L.n_chunks_p > 1 ? at<void>(ws, L.apart_p) : nullptr};
  launch_attention(ctx->dt, ap, s);
  enqueue_oproj(ctx, L, ws, L.pv, ev, hp, at<void>(ws, L.o_p), Mp, prow, s);
  HIP_TRY(hipStreamWaitEvent(sa, ctx->ev[0], 0));
  float2 *rope_rows = at<float2>(ws, L.rope_rows);
  launch_rope_rows(rope, prefix_lens, P_cap, B, S, D, rope_rows, sa);
  launch_norm_prep(ctx->dt, h_suffix, hs, ea.attn_norm, Ms, sa);
  QkvArgs qa{hs, Ms, c.rms_eps, ea.w_qkv, at<void>(ws, L.q), at<void>(ws, L.ks), at<void>(ws, L.vs), S, srow, rope,
             Hq, Hkv, D, rope_rows, ea.q_norm, ea.k_norm};
  launch_qkv(ctx->dt, qa, L.pa.qkv, sa);
  HIP_TRY(hipStreamWaitEvent(sa, ctx->ev[1], 0));
  AttnArgs as{at<void>(ws, L.q), S, 1, kp, vp, P_cap, at<void>(ws, L.ks), at<void>(ws, L.vs), S, prefix_lens, B, Hq,
              Hkv, D, L.n_chunks, L.chunk_keys, at<void>(ws, L.o), L.n_chunks > 1 ? at<void>(ws, L.apart) : nullptr};
  launch_attention(ctx->dt, as, sa);
  enqueue_mlp(ctx, L, ws, L.pv, ev, hp, at<void>(ws, L.act_p), Mp, c.vlm_ffn, prow, nullptr, s);
  Layout La = L;  // the action expert's K-split partials in a region of their own
  La.split = L.split_a;
  enqueue_finish(ctx, La, ws, L.pa, ea, hs, at<void>(ws, L.o), at<void>(ws, L.act), Ms, c.act_ffn, srow, nullptr, sa);
  HIP_TRY(hipEventRecord(ctx->ev[2], sa));
  HIP_TRY(hipStreamWaitEvent(s, ctx->ev[2], 0));
  HIP_TRY(hipGetLastError());
  return DM_OK;
}

dm_status dm_prefill_kv(dm_ctx *ctx, const dm_expert_weights *vlm, const float *prefix_embeds,
                        const int32_t *prefix_lens, int B, int P_cap, void *k_cache, void *v_cache, void *ws,
                        size_t ws_bytes, void *stream) {
  TRY(check_prefill(ctx, vlm, prefix_embeds, prefix_lens, B, P_cap, k_cache, v_cache, ws, ws_bytes));
  TRY(set_device(ctx));
  enqueue_prefill(ctx, vlm, prefix_embeds, prefix_lens, B, P_cap, k_cache, v_cache, ws, (hipStream_t)stream);
  HIP_TRY(hipGetLastError());
  return DM_OK;
}

dm_status dm_train_merged_layer(dm_ctx *ctx, const dm_expert_weights *vlm, const dm_action_weights *aw, int layer,
                                const float *h_prefix, const int32_t *prefix_lens, int B, int P_cap,
                                const float *actions, const float *noise, const float *t, const float *mask,
                                int knowledge_insulation, float *loss, const dm_train_grads *grads, void *ws,
                                size_t ws_bytes, void *stream) {
  REQUIRE(ctx, DM_ERR_INVALID_ARG, "ctx is NULL");
  const dm_config &c = ctx->cfg;
  REQUIRE(!(c.flags & (DM_FLAG_TIME_MODULATION | DM_FLAG_QK_NORM)), DM_ERR_UNSUPPORTED,
          "the training step covers the additive-time, plain-QK model (no DM_FLAG_TIME_MODULATION / DM_FLAG_QK_NORM)");
  REQUIRE(prefix_lens, DM_ERR_INVALID_ARG, "prefix_lens is NULL");
  REQUIRE(B >= 1 && B <= 4096, DM_ERR_SHAPE, "B must be 1..4096 (got %d)", B);
  REQUIRE(P_cap >= 1 && P_cap <= 65536, DM_ERR_SHAPE, "P_cap must be 1..65536 (got %d)", P_cap);
  REQUIRE(layer >= 0 && layer < c.n_layers, DM_ERR_SHAPE, "layer %d outside 0..%d", layer, c.n_layers - 1);
  TRY(check_expert(vlm, c.vlm_mlp_dtype == DM_FP8_E4M3, "VLM", false));
  TRY(check_action(ctx, aw));
  REQUIRE(h_prefix && actions && noise && t && mask && loss && grads, DM_ERR_INVALID_ARG,
          "h_prefix / actions / noise / t / mask / loss / grads is NULL");
  const dm_train_grads &G = *grads;
  const float *need[] = {G.attn_norm, G.w_qkv, G.w_o, G.mlp_norm, G.w_gate, G.w_up, G.w_down,
                         G.w_in, G.b_in, G.final_norm, G.w_out, G.b_out};
  for (const float *p : need) REQUIRE(p, DM_ERR_INVALID_ARG, "an action-side gradient pointer is NULL");
  const bool ki = knowledge_insulation != 0;
  REQUIRE(ki || (G.vlm_attn_norm && G.vlm_w_qkv), DM_ERR_INVALID_ARG,
          "without knowledge insulation vlm_attn_norm and vlm_w_qkv gradients are required");
  REQUIRE(ws, DM_ERR_INVALID_ARG, "workspace is NULL");
  REQUIRE(((uintptr_t)ws & 255u) == 0, DM_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const TrainLayout L = train_layout(c, B, P_cap);
  REQUIRE(ws_bytes >= L.total, DM_ERR_WORKSPACE, "workspace too small: %zu bytes, need %zu", ws_bytes, L.total);
  REQUIRE(ctx->side, DM_ERR_HIP, "the context has no side stream (dm_ctx_create could not make the device current)");
  TRY(set_device(ctx));
  hipStream_t s = (hipStream_t)stream;
  // Parts of the step that no later kernel on the critical path reads run on the context's side
  // stream `s2`, each after an event on `s` that marks its inputs ready: the prefix K/V
  // projection (forward), the weight gradients of the MLP and the O-projection, and the whole
  // prefix backward; `s` waits for `s2` at the end, so the step is ordered on `stream` alone.
  // Each stream has its own split-K and column-sum scratch.
  hipStream_t s2 = ctx->side;
  hipEvent_t *ev = ctx->ev;
  auto fork = [&](int k) {  // s2 waits for what s has enqueued so far
    HIP_TRY(hipEventRecord(ev[k], s));
    HIP_TRY(hipStreamWaitEvent(s2, ev[k], 0));
    return DM_OK;
  };

  const int S = c.chunk, A = c.action_dim, D = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads, grp = Hq / Hkv;
  const int Ha = c.act_hidden, Hv = c.vlm_hidden, F = c.act_ffn, QKV = (Hq + 2 * Hkv) * D, HqD = Hq * D, KV2 = 2 * Hkv * D;
  const int M = B * S, Mp = B * P_cap, T = P_cap + S, l = layer;
  const Dt dt = ctx->dt;
  const size_t es = ctx->es;
  const float eps = c.rms_eps, isd = 1.0f / sqrtf((float)D);
  const double base = c.rope_base;
  const int *lens = prefix_lens;
  auto F32 = [&](const Region &r) { return at<float>(ws, r); };
  float *x = F32(L.x), *u = F32(L.u), *v = F32(L.v), *dv = F32(L.dv), *h0 = F32(L.h0), *n1 = F32(L.n1),
        *r1 = F32(L.r1), *qkv = F32(L.qkv), *dqkv = F32(L.dqkv), *K = F32(L.K), *V = F32(L.V), *dK = F32(L.dK),
        *dV = F32(L.dV), *sc = F32(L.sc), *dp = F32(L.dp), *o = F32(L.o), *dO = F32(L.dO), *h1 = F32(L.h1),
        *n2 = F32(L.n2), *r2 = F32(L.r2), *gt = F32(L.gt), *up = F32(L.up), *act = F32(L.act), *dgt = F32(L.dgt),
        *dup = F32(L.dup), *dact = F32(L.dact), *h2 = F32(L.h2), *nf = F32(L.nf), *rf = F32(L.rf), *dnf = F32(L.dnf),
        *dh2 = F32(L.dh2), *dn2 = F32(L.dn2), *dh1 = F32(L.dh1), *dn1 = F32(L.dn1), *dh0 = F32(L.dh0),
        *np_ = F32(L.np), *rp = F32(L.rp), *kvp = F32(L.kvp), *dkvp = F32(L.dkvp), *dnp = F32(L.dnp),
        *split = F32(L.split), *cpart = F32(L.cpart), *split2 = F32(L.split2), *cpart2 = F32(L.cpart2);
  const dm_expert_weights &W = aw->body;
  const char *wq = layer_ptr(W.w_qkv, (size_t)QKV * Ha, l, es), *wo = layer_ptr(W.w_o, (size_t)Ha * HqD, l, es);
  const char *wg = layer_ptr(W.w_gate, (size_t)F * Ha, l, es), *wu = layer_ptr(W.w_up, (size_t)F * Ha, l, es);
  const char *wd = layer_ptr(W.w_down, (size_t)Ha * F, l, es);
  const char *wv_kv = layer_ptr(vlm->w_qkv, (size_t)QKV * Hv, l, es) + (size_t)HqD * Hv * es;  // K/V rows
  const float *g1 = W.attn_norm + (size_t)l * Ha, *g2 = W.mlp_norm + (size_t)l * Ha, *gv = vlm->attn_norm + (size_t)l * Hv;
  // C[M][N] = A(m, k) B(n, k) (+ C with beta 1); operands by element strides {so, si, sm, sk}
  const TOperand ROW_K = {0, 0, 0, 1};
  auto rows = [&](long ld) { TOperand t = ROW_K; t.sm = ld; return t; };     // X[m][k] row-major, row length ld
  auto cols = [&](long ld) { return TOperand{0, 0, 1, ld}; };                 // X[k][m] read as (m, k)
  auto mm_on = [&](hipStream_t st, int Mm, int Nn, int Kk, TOperand a, Dt ta, const void *pa, TOperand b, Dt tb,
                   const void *pb, float *C, long ldc, float beta = 0.f) {
    TGemm g{};
    g.M = Mm, g.N = Nn, g.K = Kk, g.a = a, g.b = b, g.bdiv = 1, g.C = C, g.ldc = ldc, g.zo_n = 1, g.zi_n = 1;
    g.alpha = 1.f, g.beta = beta, g.part = st == s ? split : split2, g.part_floats = kTrainSplitFloats;
    launch_tgemm(g, ta, pa, tb, pb, st);
  };
  auto mm = [&](int Mm, int Nn, int Kk, TOperand a, Dt ta, const void *pa, TOperand b, Dt tb, const void *pb,
                float *C, long ldc, float beta = 0.f) { mm_on(s, Mm, Nn, Kk, a, ta, pa, b, tb, pb, C, ldc, beta); };
  auto colsum = [&](const float *dy, const float *xx, const float *rr, int Mm, int Nn, float *out) {
    launch_colsum(dy, xx, rr, Mm, Nn, out, cpart, s);
  };

  // ---- forward
  // prefix (side stream): the VLM expert's pre-norm and K/V rows (rows past each prefix are
  // zero), RoPE on K
  TRY(fork(0));
  launch_rms_fwd(h_prefix, DT_F32, gv, eps, Mp, Hv, lens, P_cap, np_, rp, s2);
  mm_on(s2, Mp, KV2, Hv, rows(Hv), DT_F32, np_, rows(Hv), dt, wv_kv, kvp, KV2);
  launch_rope_rows(kvp, Mp, P_cap, KV2, 0, Hkv, D, base, lens, false, 1.0f, s2);
  HIP_TRY(hipEventRecord(ev[1], s2));
  launch_fm_embed(actions, noise, t, aw->w_in, aw->b_in, B, S, A, Ha, 10000.0f, x, u, h0, s);
  // action rows: pre-norm, Q/K/V, RoPE on Q and K at positions P_b + s
  launch_rms_fwd(h0, DT_F32, g1, eps, M, Ha, nullptr, 1, n1, r1, s);
  mm(M, QKV, Ha, rows(Ha), DT_F32, n1, rows(Ha), dt, wq, qkv, QKV);
  launch_rope_rows(qkv, M, S, QKV, 0, Hq + Hkv, D, base, lens, true, 1.0f, s);
  HIP_TRY(hipStreamWaitEvent(s, ev[1], 0));
  launch_gather_kv(kvp, qkv, lens, B, P_cap, S, Hq, Hkv, D, K, V, s);
  // scores[b][h][s][j] = q . k / sqrt(D), softmax over the visible keys, O = P V
  TGemm at_{};
  at_.zo_n = B, at_.zi_n = Hq, at_.bdiv = grp, at_.alpha = 1.f, at_.part = split, at_.part_floats = kTrainSplitFloats;
  {
    TGemm g = at_;
    g.M = S, g.N = T, g.K = D, g.alpha = isd;
    g.a = {(long)S * QKV, D, QKV, 1};
    g.b = {(long)Hkv * T * D, (long)T * D, D, 1};
    g.C = sc, g.ldc = T, g.c_so = (long)Hq * S * T, g.c_si = (long)S * T;
    launch_tgemm(g, DT_F32, qkv, DT_F32, K, s);
  }
  launch_softmax_rows(sc, lens, B, Hq, S, P_cap, s);
  {
    TGemm g = at_;
    g.M = S, g.N = D, g.K = T;
    g.a = {(long)Hq * S * T, (long)S * T, T, 1};
    g.b = {(long)Hkv * T * D, (long)T * D, 1, D};
    g.C = o, g.ldc = HqD, g.c_so = (long)S * HqD, g.c_si = D;
    launch_tgemm(g, DT_F32, sc, DT_F32, V, s);
  }
  launch_copy_bias(h0, nullptr, M, Ha, h1, s);
  mm(M, Ha, HqD, rows(HqD), DT_F32, o, rows(HqD), dt, wo, h1, Ha, 1.f);
  launch_rms_fwd(h1, DT_F32, g2, eps, M, Ha, nullptr, 1, n2, r2, s);
  mm(M, F, Ha, rows(Ha), DT_F32, n2, rows(Ha), dt, wg, gt, F);
  mm(M, F, Ha, rows(Ha), DT_F32, n2, rows(Ha), dt, wu, up, F);
  launch_swiglu_fwd(gt, up, (long)M * F, act, s);
  launch_copy_bias(h1, nullptr, M, Ha, h2, s);
  mm(M, Ha, F, rows(F), DT_F32, act, rows(F), dt, wd, h2, Ha, 1.f);
  launch_rms_fwd(h2, DT_F32, aw->final_norm, eps, M, Ha, nullptr, 1, nf, rf, s);
  launch_copy_bias(nullptr, aw->b_out, M, A, v, s);
  mm(M, A, Ha, rows(Ha), DT_F32, nf, rows(Ha), DT_F32, aw->w_out, v, A, 1.f);
  launch_fm_loss(v, u, mask, (long)M * A, loss, dv, s);

  // ---- backward: head, final norm
  mm(A, Ha, M, cols(A), DT_F32, dv, cols(Ha), DT_F32, nf, G.w_out, Ha);
  colsum(dv, nullptr, nullptr, M, A, G.b_out);
  mm(M, Ha, A, rows(A), DT_F32, dv, cols(Ha), DT_F32, aw->w_out, dnf, Ha);
  launch_rms_bwd(h2, DT_F32, aw->final_norm, dnf, rf, nullptr, M, Ha, dh2, s);
  colsum(dnf, h2, rf, M, Ha, G.final_norm);
  // MLP (its weight gradients on the side stream: nothing on `s` reads them)
  TRY(fork(2));
  mm_on(s2, Ha, F, M, cols(Ha), DT_F32, dh2, cols(F), DT_F32, act, G.w_down, F);
  mm(M, F, Ha, rows(Ha), DT_F32, dh2, cols(F), dt, wd, dact, F);
  launch_swiglu_bwd(gt, up, dact, (long)M * F, dgt, dup, s);
  TRY(fork(3));
  mm_on(s2, F, Ha, M, cols(F), DT_F32, dgt, cols(Ha), DT_F32, n2, G.w_gate, Ha);
  mm_on(s2, F, Ha, M, cols(F), DT_F32, dup, cols(Ha), DT_F32, n2, G.w_up, Ha);
  mm(M, Ha, F, rows(F), DT_F32, dgt, cols(Ha), dt, wg, dn2, Ha);
  mm(M, Ha, F, rows(F), DT_F32, dup, cols(Ha), dt, wu, dn2, Ha, 1.f);
  launch_rms_bwd(h1, DT_F32, g2, dn2, r2, dh2, M, Ha, dh1, s);
  colsum(dn2, h1, r2, M, Ha, G.mlp_norm);
  // O-projection (weight gradient on the side stream)
  TRY(fork(4));
  mm_on(s2, Ha, HqD, M, cols(Ha), DT_F32, dh1, cols(HqD), DT_F32, o, G.w_o, HqD);
  mm(M, HqD, Ha, rows(Ha), DT_F32, dh1, cols(HqD), dt, wo, dO, HqD);
  // attention: dP = dO V^T, dS = P (dP - rowsum(P dP)) / sqrt(D), dQ = dS K, dK = dS^T Q, dV = P^T dO
  {
    TGemm g = at_;
    g.M = S, g.N = T, g.K = D;
    g.a = {(long)S * HqD, D, HqD, 1};
    g.b = {(long)Hkv * T * D, (long)T * D, D, 1};
    g.C = dp, g.ldc = T, g.c_so = (long)Hq * S * T, g.c_si = (long)S * T;
    launch_tgemm(g, DT_F32, dO, DT_F32, V, s);
  }
  launch_softmax_bwd(sc, dp, (long)B * Hq * S, T, isd, s);
  {
    TGemm g = at_;
    g.M = S, g.N = D, g.K = T;
    g.a = {(long)Hq * S * T, (long)S * T, T, 1};
    g.b = {(long)Hkv * T * D, (long)T * D, 1, D};
    g.C = dqkv, g.ldc = QKV, g.c_so = (long)S * QKV, g.c_si = D;
    launch_tgemm(g, DT_F32, dp, DT_F32, K, s);
  }
  for (int r = 0; r < grp; ++r) {  // the grp query heads of a KV head add into its dK / dV
    TGemm g{};
    g.M = T, g.N = D, g.K = S, g.bdiv = 1, g.zo_n = B, g.zi_n = Hkv, g.alpha = 1.f, g.beta = r ? 1.f : 0.f;
    g.part = split, g.part_floats = kTrainSplitFloats;
    g.ldc = D, g.c_so = (long)Hkv * T * D, g.c_si = (long)T * D;
    g.a = {(long)Hq * S * T, (long)grp * S * T, 1, T};
    g.b = {(long)S * QKV, (long)grp * D, 1, QKV};
    g.C = dK;
    launch_tgemm(g, DT_F32, dp + (size_t)r * S * T, DT_F32, qkv + (size_t)r * D, s);
    g.b = {(long)S * HqD, (long)grp * D, 1, HqD};
    g.C = dV;
    launch_tgemm(g, DT_F32, sc + (size_t)r * S * T, DT_F32, dO + (size_t)r * D, s);
  }
  launch_scatter_kv(dK, dV, lens, B, P_cap, S, Hq, Hkv, D, dqkv, ki ? nullptr : dkvp, s);
  // the VLM side (side stream): through the prefix K/V, or nothing with knowledge insulation
  TRY(fork(5));
  if (ki) {
    if (G.vlm_attn_norm) launch_fill(G.vlm_attn_norm, Hv, 0.f, s2);
    if (G.vlm_w_qkv) launch_fill(G.vlm_w_qkv, (long)QKV * Hv, 0.f, s2);
    if (G.h_prefix) launch_fill(G.h_prefix, (long)Mp * Hv, 0.f, s2);
  } else {
    launch_rope_rows(dkvp, Mp, P_cap, KV2, 0, Hkv, D, base, lens, false, -1.0f, s2);
    launch_fill(G.vlm_w_qkv, (long)HqD * Hv, 0.f, s2);  // the query rows do not reach the loss
    mm_on(s2, KV2, Hv, Mp, cols(KV2), DT_F32, dkvp, cols(Hv), DT_F32, np_, G.vlm_w_qkv + (size_t)HqD * Hv, Hv);
    mm_on(s2, Mp, Hv, KV2, rows(KV2), DT_F32, dkvp, cols(Hv), dt, wv_kv, dnp, Hv);
    if (G.h_prefix) launch_rms_bwd(h_prefix, DT_F32, gv, dnp, rp, nullptr, Mp, Hv, G.h_prefix, s2);
    launch_colsum(dnp, h_prefix, rp, Mp, Hv, G.vlm_attn_norm, cpart2, s2);
  }
  HIP_TRY(hipEventRecord(ev[6], s2));
  launch_rope_rows(dqkv, M, S, QKV, 0, Hq + Hkv, D, base, lens, true, -1.0f, s);
  // Q/K/V projection and the attention pre-norm
  mm(QKV, Ha, M, cols(QKV), DT_F32, dqkv, cols(Ha), DT_F32, n1, G.w_qkv, Ha);
  mm(M, Ha, QKV, rows(QKV), DT_F32, dqkv, cols(Ha), dt, wq, dn1, Ha);
  launch_rms_bwd(h0, DT_F32, g1, dn1, r1, dh1, M, Ha, dh0, s);
  colsum(dn1, h0, r1, M, Ha, G.attn_norm);
  // action_in_proj
  mm(Ha, A, M, cols(Ha), DT_F32, dh0, cols(A), DT_F32, x, G.w_in, A);
  colsum(dh0, nullptr, nullptr, M, Ha, G.b_in);
  HIP_TRY(hipStreamWaitEvent(s, ev[6], 0));  // join the side stream
  HIP_TRY(hipGetLastError());
  return DM_OK;
}

dm_status dm_quantize_fp8_rows(const void *src, uint8_t *dst, float *scales, int rows, int cols, void *stream) {
  REQUIRE(src && dst && scales, DM_ERR_INVALID_ARG, "src / dst / scales is NULL");
  REQUIRE(rows >= 1 && cols >= 1, DM_ERR_SHAPE, "rows and cols must be positive");
  REQUIRE(aligned16(src) && aligned16(dst), DM_ERR_INVALID_ARG, "src and dst must be 16-byte aligned");
  // run on the device that holds the data (there is no context to name it)
  hipPointerAttribute_t attr;
  HIP_TRY(hipPointerGetAttributes(&attr, src));
  REQUIRE(attr.type == hipMemoryTypeDevice, DM_ERR_INVALID_ARG, "src is not device memory");
  int cur = -1;
  HIP_TRY(hipGetDevice(&cur));
  if (cur != attr.device) HIP_TRY(hipSetDevice(attr.device));
  launch_fp8_quantize_rows(src, dst, scales, rows, cols, (hipStream_t)stream);
  HIP_TRY(hipGetLastError());
  return DM_OK;
}

}  // extern "C"

// Merged grouped-query attention on gfx950 MFMA.
// Page "DM0 paper definition vs. Dexbotic code", section 1: the two experts' Q/K/V are joined
// along the sequence for one attention (16 query heads over 8 KV heads).  With the block mask,
// a prefix query sees the sample's P_b prefix keys and an action query sees those plus all S
// action keys; page "DM0.5: High-Performance Embodied VLA ...", section 5.1: the prefix keys
// are the cached VLM K/V, so the kernel streams them straight from the cache layout
// [B][Hkv][P_cap][D] followed by the action keys [B][Hkv][S][D], never concatenating them.
//
// One 512-thread workgroup takes one (sample, KV head, query block, key chunk): 128 query
// slots = the G query heads of the KV head x 128/G query rows.  Its 8 waves form 4 slot groups of
// 32 slots x 2 key halves: both waves of a pair see every LDS stage, each takes one half of every
// 64-key tile with its own online softmax, and the pair merges (max, sum, output) through LDS at
// the end.  Two waves per SIMD hide each other's LDS and MFMA latencies while every K/V byte is
// still read from LDS only once per slot group.  Two kernels share this work split:
// attn_dma_kernel (bf16, head dim 128, the DM0 shapes; described at its definition) copies the
// operands into LDS by DMA, several stages ahead; attn_kernel (other head dims, fp32) stages
// keys through LDS 128 at a time (K row-major, V transposed) from registers, every load of a
// stage issued before the first is consumed, the next stage loaded while the current one is
// multiplied.  Scores are formed transposed,
// S^T = K Q^T, so every lane owns one query column: the online-softmax statistics stay in-lane
// (plus two cross-lane-group exchanges) and the probabilities already sit in the B-operand
// layout of O^T = V^T P^T.  The key rows of each 16-key score tile are permuted so a lane's
// probabilities are consecutive keys of the next MFMA's contraction chunk.  Softmax is float32
// with base-2 exponentials; the running output is rescaled only when some column's maximum grew.
// With several key chunks, each workgroup stores its normalised partial output (weight dtype)
// with its running max and sum, and attn_combine_kernel merges them in chunk order.
#include "common.h"
#include "kernels.h"

namespace dm {

constexpr int ATT_SLOTS = 128;
constexpr int ATT_KT = 64;    // keys per tile (32 per wave of a pair)
constexpr int ATT_CH = 128;   // keys staged in LDS per pass
constexpr int ATT_THREADS = 512;

int attn_qblocks(int q_rows, int Hq, int Hkv) {
  const int rph = ATT_SLOTS / (Hq / Hkv);
  return (q_rows + rph - 1) / rph;
}
__host__ __device__ static size_t part_o_elems(int B, int Hkv, int nqb, int n_chunks, int D) {
  return (size_t)B * Hkv * nqb * n_chunks * ATT_SLOTS * D;
}
size_t attn_partial_bytes(Dt dt, int B, int Hkv, int nqb, int n_chunks, int D) {
  const size_t o = part_o_elems(B, Hkv, nqb, n_chunks, D) * (dt == DT_BF16 ? 2 : 4);
  const size_t ml = (size_t)B * Hkv * nqb * n_chunks * ATT_SLOTS * 2 * sizeof(float);
  return ((o + 255) & ~(size_t)255) + ml;
}

// 4 consecutive output values of one lane: one 8-byte (bf16) or 16-byte (fp32) store.
template <typename T> __device__ __forceinline__ void store4(T *p, f32x4 v, float s);
template <> __device__ __forceinline__ void store4<bf16>(bf16 *p, f32x4 v, float s) {
  bf16x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (bf16)(v[i] * s);
  *reinterpret_cast<bf16x4 *>(p) = o;
}
template <> __device__ __forceinline__ void store4<float>(float *p, f32x4 v, float s) {
  *reinterpret_cast<f32x4 *>(p) = v * s;
}

// Merge the two key halves of every slot group (the second wave of a pair hands its state over
// through the LDS, which must be free by now), then write the normalised output, or, with several
// key chunks, this chunk's normalised partial output and its (max, sum); a chunk past the
// sample's keys publishes max -inf and sum 0 (weight 0 in the merge).
// Lane (g, c16) holds O^T rows dt*16 + 4g .. +3 of query column c16: 4 consecutive outputs.
template <typename T, int D>
__device__ __forceinline__ void attn_finish(const AttnArgs &a, char *smem, float (&m)[2], float (&l)[2],
                                            f32x4 (&o)[2][D / 16], int wave, int lane, int b, int h, int r0, int nq,
                                            size_t grp, int chunk, int nch) {
  constexpr int DT = D / 16;
  constexpr int XO = 4 * 2 * DT * 64;  // float4 outputs of the second waves
  const int sg = wave & 3, kh = wave >> 2, g = lane >> 4, c16 = lane & 15;
  float *xo = reinterpret_cast<float *>(smem);
  float *xm = xo + XO * 4, *xl = xm + 4 * 2 * 64;
  if (kh == 1) {
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4 *>(&xo[(((sg * 2 + qt) * DT + dt) * 64 + lane) * 4]) = o[qt][dt];
      xm[(sg * 2 + qt) * 64 + lane] = m[qt];
      xl[(sg * 2 + qt) * 64 + lane] = l[qt];
    }
  }
  __syncthreads();
  if (kh == 1) return;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float m1 = xm[(sg * 2 + qt) * 64 + lane], l1 = xl[(sg * 2 + qt) * 64 + lane];
    const float M = fmaxf(m[qt], m1);
    const float Mu = M == -INFINITY ? 0.f : M;
    const float a0 = __builtin_amdgcn_exp2f(m[qt] - Mu), a1 = __builtin_amdgcn_exp2f(m1 - Mu);
    l[qt] = l[qt] * a0 + l1 * a1;
    m[qt] = M;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      o[qt][dt] = o[qt][dt] * a0 + *reinterpret_cast<const f32x4 *>(&xo[(((sg * 2 + qt) * DT + dt) * 64 + lane) * 4]) * a1;
  }

  const int HD = a.Hq * D;
  if (a.n_chunks == 1) {
    T *out = (T *)a.out;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int row = r0 + qt * 16 + c16;
      if (row >= nq) continue;
      const float inv = 1.0f / l[qt];
      T *orow = out + (size_t)(b * a.q_rows_per_b + row) * HD + h * D + 4 * g;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) store4<T>(orow + dt * 16, o[qt][dt], inv);
    }
    return;
  }
  const int nqb = gridDim.y, slot0 = sg * 32;
  T *part_o = (T *)a.part;
  float *part_ml = (float *)((char *)a.part + ((part_o_elems(a.B, a.Hkv, nqb, a.n_chunks, D) * sizeof(T) + 255) &
                                               ~(size_t)255));
  T *po = part_o + (grp * a.n_chunks + chunk) * ATT_SLOTS * D;
  float *pml = part_ml + (grp * a.n_chunks + chunk) * ATT_SLOTS * 2;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int row = r0 + qt * 16 + c16;
    if (row >= nq) continue;
    const int slot = slot0 + qt * 16 + c16;
    if (chunk < nch) {
      const float inv = 1.0f / l[qt];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) store4<T>(po + slot * D + dt * 16 + 4 * g, o[qt][dt], inv);
    }
    if (g == 0) *reinterpret_cast<float2 *>(&pml[slot * 2]) = chunk < nch ? make_float2(m[qt], l[qt]) : make_float2(-INFINITY, 0.f);
  }
}

template <typename T, int D, int G>
__global__ __launch_bounds__(ATT_THREADS) void attn_kernel(AttnArgs a) {
  typedef Mfma<T> MF;
  typedef typename MF::frag frag;
  constexpr int EPL = MF::EPL, KC = 4 * EPL;
  constexpr int DC = D / KC;        // contraction chunks of Q K^T
  constexpr int DT = D / 16;        // 16-row tiles of O^T
  constexpr int HK = ATT_KT / 2;    // keys of a tile per wave
  constexpr int NPV = HK / KC;      // contraction chunks of V^T P^T per half tile
  constexpr int SUB = EPL / 4;      // 16-key score tiles per P^T chunk
  constexpr int NS = HK / 16;       // 16-key score tiles per half tile
  constexpr int RPH = ATT_SLOTS / G;
  constexpr int KLD = D + EPL, VLD = ATT_CH + EPL;
  constexpr int VPRW = D / EPL;                      // 16-byte vectors per key row
  constexpr int LPT = ATT_CH * VPRW / ATT_THREADS;   // vectors per thread per stage
  constexpr int STAGE_B = (ATT_CH * KLD + D * VLD) * (int)sizeof(T);
  constexpr int XO = 4 * 2 * DT * 64;                // merge: float4 outputs of the second waves
  constexpr int MERGE_B = XO * 16 + 2 * 4 * 2 * 64 * 4;
  __shared__ __attribute__((aligned(16))) char smem[STAGE_B > MERGE_B ? STAGE_B : MERGE_B];
  T *Ks = reinterpret_cast<T *>(smem);
  T *Vt = Ks + ATT_CH * KLD;

  const T *__restrict__ q = (const T *)a.q;
  const T *__restrict__ kp = (const T *)a.kp;
  const T *__restrict__ vp = (const T *)a.vp;
  const T *__restrict__ ks = (const T *)a.ks;
  const T *__restrict__ vs = (const T *)a.vs;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sg = wave & 3, kh = wave >> 2;  // slot group, key half
  const int g = lane >> 4, c16 = lane & 15;
  const int bk = blockIdx.x, qb = blockIdx.y, chunk = blockIdx.z, nqb = gridDim.y;
  const int b = bk / a.Hkv, kvh = bk - b * a.Hkv;
  const int P = max(0, min(a.lens[b], a.kp_rows));
  const int nq = a.suffix ? a.S : P;
  const int nkeys = P + (a.suffix ? a.S : 0);
  const int nch = (nkeys + a.chunk_keys - 1) / a.chunk_keys;  // chunks holding keys
  const int k_begin = chunk * a.chunk_keys;
  const int k_end = min(nkeys, k_begin + a.chunk_keys);
  if (qb * RPH >= nq) return;  // no query rows here: uniform, and no merge is needed

  const int slot0 = sg * 32;
  const int h = kvh * G + slot0 / RPH;
  const int r0 = qb * RPH + (slot0 % RPH);
  const int HD = a.Hq * D;
  const size_t grp = (size_t)bk * nqb + qb;

  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  f32x4 o[2][DT];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (k_begin < k_end) {
    frag qf[2][DC];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int row = r0 + qt * 16 + c16;
      // rows past nq read row nq-1: their columns of the score tile are never stored
      const T *qrow = q + (size_t)(b * a.q_rows_per_b + min(row, nq - 1)) * HD + h * D;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) qf[qt][dc] = load_frag<T>(qrow + dc * KC + g * EPL);
    }
    const float sc = 1.4426950408889634f / sqrtf((float)D);  // log2(e) / sqrt(D)
    const size_t pre_base = (size_t)(b * a.Hkv + kvh) * a.kp_rows * D;
    const size_t suf_base = (size_t)(b * a.Hkv + kvh) * a.S * D;

    // K: 16-byte vectors, lanes along a row (coalesced).  V: lanes along keys, so the transposed
    // LDS stores of a wave hit consecutive addresses.  Keys past k_end re-read key k_end-1: their
    // scores are masked to -inf and their V rows are finite, so they add exactly 0.
    frag kv[LPT], vv[LPT];
    auto stage_load = [&](int ks0) {
#pragma unroll
      for (int v = 0; v < LPT; ++v) {
        const int idx = tid + v * ATT_THREADS;
        const int r = idx / VPRW, cv = idx - r * VPRW;
        const int kc = min(ks0 + r, k_end - 1);
        const size_t off = kc < P ? pre_base + (size_t)kc * D : suf_base + (size_t)(kc - P) * D;
        kv[v] = load_frag<T>((kc < P ? kp : ks) + off + cv * EPL);
      }
#pragma unroll
      for (int v = 0; v < LPT; ++v) {
        const int idx = tid + v * ATT_THREADS;
        const int cv = idx / ATT_CH, r = idx - cv * ATT_CH;
        const int kc = min(ks0 + r, k_end - 1);
        const size_t off = kc < P ? pre_base + (size_t)kc * D : suf_base + (size_t)(kc - P) * D;
        vv[v] = load_frag<T>((kc < P ? vp : vs) + off + cv * EPL);
      }
    };
    stage_load(k_begin);
    for (int ks0 = k_begin; ks0 < k_end; ks0 += ATT_CH) {
      __syncthreads();  // the previous stage is consumed
#pragma unroll
      for (int v = 0; v < LPT; ++v) {
        const int idx = tid + v * ATT_THREADS;
        const int r = idx / VPRW, cv = idx - r * VPRW;
        *reinterpret_cast<frag *>(&Ks[r * KLD + cv * EPL]) = kv[v];
      }
#pragma unroll
      for (int v = 0; v < LPT; ++v) {
        const int idx = tid + v * ATT_THREADS;
        const int cv = idx / ATT_CH, r = idx - cv * ATT_CH;
#pragma unroll
        for (int e = 0; e < EPL; ++e) Vt[(cv * EPL + e) * VLD + r] = vv[v][e];
      }
      __syncthreads();
      if (ks0 + ATT_CH < k_end) stage_load(ks0 + ATT_CH);

      const int stage_keys = min(ATT_CH, k_end - ks0);
      for (int t0 = kh * HK; t0 < stage_keys; t0 += ATT_KT) {  // this wave's half of every tile
        // scores S^T for NS 16-key tiles x both 16-slot halves; each K fragment read once
        f32x4 st[2][NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int pv = s / SUB, kk = s % SUB;
          const int krow = t0 + pv * KC + (c16 >> 2) * EPL + 4 * kk + (c16 & 3);
          frag kf[DC];
#pragma unroll
          for (int dc = 0; dc < DC; ++dc) kf[dc] = *reinterpret_cast<const frag *>(&Ks[krow * KLD + dc * KC + g * EPL]);
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dc = 0; dc < DC; ++dc) acc = MF::mma(kf[dc], qf[qt][dc], acc);
            st[qt][s] = acc;
          }
        }
        const bool partial = ks0 + t0 + HK > k_end;  // uniform: only the last tile masks keys
        frag pf[2][NPV];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          if (partial) {
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (ks0 + t0 + (s / SUB) * KC + g * EPL + 4 * (s % SUB) + i >= k_end) st[qt][s][i] = -INFINITY;
          }
          float mx = st[qt][0][0];
#pragma unroll
          for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, st[qt][s][i]);
          mx = max_xor32(max_xor16(mx)) * sc;
          const float m_new = fmaxf(m[qt], mx);
          const float m_use = m_new == -INFINITY ? 0.f : m_new;
          float sum = 0.f;
#pragma unroll
          for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float p = __builtin_amdgcn_exp2f(fmaf(st[qt][s][i], sc, -m_use));
              st[qt][s][i] = p;
              sum += p;
            }
          sum = sum_xor32(sum_xor16(sum));
          // rescale only when some column's maximum grew (wave-uniform branch)
          if (__ballot(m_new > m[qt]) != 0) {
            const float alpha = __builtin_amdgcn_exp2f(m[qt] - m_use);
            l[qt] *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[qt][dt] *= alpha;
          }
          l[qt] += sum;
          m[qt] = m_new;
#pragma unroll
          for (int pv = 0; pv < NPV; ++pv)
#pragma unroll
            for (int kk = 0; kk < SUB; ++kk)
#pragma unroll
              for (int i = 0; i < 4; ++i) pf[qt][pv][kk * 4 + i] = from_f32<T>(st[qt][pv * SUB + kk][i]);
        }
        // O^T += V^T P^T; each V fragment read once for both halves
#pragma unroll
        for (int pv = 0; pv < NPV; ++pv)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const frag vf = *reinterpret_cast<const frag *>(&Vt[(dt * 16 + c16) * VLD + t0 + pv * KC + g * EPL]);
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) o[qt][dt] = MF::mma(vf, pf[qt][pv], o[qt][dt]);
          }
      }
    }
  }

  __syncthreads();  // every stage read is done: the LDS is free
  attn_finish<T, D>(a, smem, m, l, o, wave, lane, b, h, r0, nq, grp, chunk, nch);
}

// ------------------------------------------------------------------ bf16, head_dim 128
// The same work split (8 waves = 4 slot groups x 2 key halves, 64-key tiles, online softmax per
// wave, pair merge), with the operands copied global -> LDS by the DMA path
// (global_load_lds_dwordx4): the query tile and NBUF-1 key stages are in flight before the first
// tile is multiplied, and every iteration starts the copy of the stage NBUF-1 ahead, so about
// 96 KB per workgroup stay in flight and the kernel streams the cache at the HBM rate instead of
// one load round trip per stage.  K and V stay row-major in LDS (256-byte rows): V^T fragments
// are read with the gfx950 transposing LDS read (ds_read_b64_tr_b16), so no register staging
// or transposed LDS stores are needed.
//
// LDS rows of 256 bytes keep their 16-byte chunks permuted: chunk c of row r sits at position
// c ^ att_swz(r).  Every read below is then free of bank conflicts: a K fragment read (16 lanes:
// 16 key rows, one chunk), a transposed V read (32 lanes: 8 key rows x 2 chunks) and a Q
// fragment read (16 consecutive slots, one chunk).
__device__ __forceinline__ int att_swz(int r) { return ((r & 3) << 1) | (r & 8) | (((r >> 4) ^ (r >> 2)) & 1); }

typedef short att_s4 __attribute__((ext_vector_type(4)));
typedef short att_s8 __attribute__((ext_vector_type(8)));
// Transposing LDS read, per group of 16 lanes: lane i receives element i % 4 of the 4-element
// (8-byte) row addressed by lane 4e + i / 4 of its group, for e = 0..3.
__device__ __forceinline__ att_s4 lds_read_tr16(const char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) att_s4 *)p);
}
__device__ __forceinline__ void vm_wait_upto12(int n) {  // n in {0, 4, 8, 12}
  if (n >= 12) vm_wait<12>();
  else if (n >= 8) vm_wait<8>();
  else if (n >= 4) vm_wait<4>();
  else vm_wait<0>();
}

template <int G, int NBUF>
__global__ __launch_bounds__(ATT_THREADS) void attn_dma_kernel(AttnArgs a) {
  typedef bf16x8 frag;
  constexpr int D = 128, DC = 4, DT = 8, RB = D * 2;  // RB: bytes per K / V / Q row
  constexpr int TK = ATT_KT;                           // keys per stage (32 per wave of a pair)
  constexpr int KV_B = TK * RB;                        // 16 KB of K, then 16 KB of V
  constexpr int STAGE = 2 * KV_B;
  constexpr int LPW = STAGE / 1024 / (ATT_THREADS / 64);  // 1 KB copies per wave per stage
  constexpr int RPH = ATT_SLOTS / G;
  static_assert(LPW == 4 && ATT_SLOTS * RB == STAGE, "the query tile fills one stage buffer");
  static_assert(NBUF >= 3 && NBUF <= 4 && NBUF * STAGE <= 160 * 1024, "stage buffers fit the LDS");
  static_assert(4 * 2 * DT * 64 * 16 + 2 * 4 * 2 * 64 * 4 <= NBUF * STAGE, "the pair merge fits the LDS");
  __shared__ __attribute__((aligned(1024))) char smem[NBUF * STAGE];

  const bf16 *__restrict__ q = (const bf16 *)a.q;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sg = wave & 3, kh = wave >> 2;
  const int g = lane >> 4, c16 = lane & 15;
  const int bk = blockIdx.x, qb = blockIdx.y, chunk = blockIdx.z, nqb = gridDim.y;
  const int b = bk / a.Hkv, kvh = bk - b * a.Hkv;
  const int P = max(0, min(a.lens[b], a.kp_rows));
  const int nq = a.suffix ? a.S : P;
  const int nkeys = P + (a.suffix ? a.S : 0);
  const int nch = (nkeys + a.chunk_keys - 1) / a.chunk_keys;
  const int k_begin = chunk * a.chunk_keys;
  const int k_end = min(nkeys, k_begin + a.chunk_keys);
  if (qb * RPH >= nq) return;  // uniform

  const int slot0 = sg * 32;
  const int h = kvh * G + slot0 / RPH;
  const int r0 = qb * RPH + (slot0 % RPH);
  const int HD = a.Hq * D;
  const size_t grp = (size_t)bk * nqb + qb;

  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  f32x4 o[2][DT];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (k_begin < k_end) {
    const unsigned sbase = lds_addr(smem);
    const int crow = lane >> 4, cpos = lane & 15;  // a copy: 4 rows x 16 chunks, one per lane
    // Stage copies: waves 0-3 copy K, waves 4-7 V; copy i of a wave fills rows 4u .. 4u+3 of the
    // stage, u = 4 (wave & 3) + i.  Keys past k_end re-read key k_end-1: their scores are masked
    // to -inf and their V rows are finite, so they add exactly 0.
    const bf16 *kv_pre = (const bf16 *)(wave < 4 ? a.kp : a.vp) + (size_t)(b * a.Hkv + kvh) * a.kp_rows * D;
    const bf16 *kv_suf = (const bf16 *)(wave < 4 ? a.ks : a.vs) + (size_t)(b * a.Hkv + kvh) * a.S * D;
    int coff[4];  // byte offsets of this lane's pieces within a stage's rows
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * (4 * (wave & 3) + i) + crow;
      coff[i] = (row * D + ((cpos ^ att_swz(row)) << 3)) * 2;
    }
    const int pre_end = min(P, k_end);
    auto issue = [&](int stage) {
      const int ks0 = k_begin + stage * TK;
      const unsigned dst = sbase + (stage % NBUF) * STAGE + (wave >> 2) * KV_B + (wave & 3) * 4 * 1024;
      if (ks0 + TK <= pre_end) {  // uniform: 64 consecutive cached keys, one scalar base
        const char *base = (const char *)(kv_pre + (size_t)ks0 * D);
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16_sbase(base, coff[i], dst + i * 1024);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 4 * (4 * (wave & 3) + i) + crow;
          const int kc = min(ks0 + row, k_end - 1);
          const bf16 *src = kc < P ? kv_pre + (size_t)kc * D : kv_suf + (size_t)(kc - P) * D;
          dma16(src + ((cpos ^ att_swz(row)) << 3), dst + i * 1024);
        }
      }
    };
    // Query tile into the last buffer (first overwritten by the stage NBUF-1 copies, which start
    // after every wave has read its fragments): copy i of a wave fills slots 4u .. 4u+3,
    // u = 4 wave + i; rows past nq read row nq-1 (their outputs are never stored).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = 4 * (4 * wave + i) + crow;
      const int row = min(qb * RPH + slot % RPH, nq - 1);
      const bf16 *src = q + (size_t)(b * a.q_rows_per_b + row) * HD + (kvh * G + slot / RPH) * D;
      dma16(src + ((cpos ^ att_swz(slot)) << 3), sbase + (NBUF - 1) * STAGE + (4 * wave + i) * 1024);
    }
    const int nt = (k_end - k_begin + TK - 1) / TK;
#pragma unroll
    for (int st = 0; st < NBUF - 1; ++st)
      if (st < nt) issue(st);
    vm_wait_upto12(min(NBUF - 2, nt - 1) * LPW);  // this wave's query and stage-0 copies have landed
    wg_barrier();
    frag qf[2][DC];
    {
      const char *Qb = smem + (NBUF - 1) * STAGE;
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const int slot = slot0 + qt * 16 + c16;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
          qf[qt][dc] = *reinterpret_cast<const frag *>(Qb + slot * RB + (((dc * 4 + g) ^ att_swz(slot)) << 4));
      }
    }
    const float sc = 1.4426950408889634f / sqrtf((float)D);  // log2(e) / sqrt(D)

    // per-lane LDS offsets within a stage (the same for every stage):
    // K fragment rows of score tile s: keys (c16 / 4) * 8 + c16 % 4 + 4 s of this wave's half,
    // so that output row 4g + i of tile s is key 8g + 4s + i (consecutive keys per lane for P^T)
    int koff[2][DC];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kr = kh * 32 + (c16 >> 2) * 8 + (c16 & 3) + 4 * s;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) koff[s][dc] = kr * RB + (((dc * 4 + g) ^ att_swz(kr)) << 4);
    }
    // V^T fragment (d = 16 dt + c16, keys 8g .. 8g+7 of the half): two transposing reads of the
    // 8-byte pieces (key 8g + j + 4 half, d = 16 dt + 4 (c16 % 4) .. +3), j = c16 / 4
    const int vr = kh * 32 + g * 8 + (c16 >> 2);
    const int vsw0 = att_swz(vr), vsw1 = att_swz(vr + 4);
    const int vpiece = (c16 >> 1) & 1, vbyte = (c16 & 1) * 8;

    // S^T of this wave's half of tile t (two 16-key score tiles x two 16-slot halves)
    auto scores = [&](int t, f32x4(&st)[2][2]) {
      const char *Kb = smem + (t % NBUF) * STAGE;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        frag kf[DC];
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) kf[dc] = *reinterpret_cast<const frag *>(Kb + koff[s][dc]);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int dc = 0; dc < DC; ++dc) acc = Mfma<bf16>::mma(kf[dc], qf[qt][dc], acc);
          st[qt][s] = acc;
        }
      }
    };
    // probabilities of tile t (relative to the column maxima mu), the lane's share of the row sums,
    // and O^T += V^T P^T
    auto exp_pv = [&](int t, f32x4(&st)[2][2], const float(&mu)[2]) {
      frag pf[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        float sum = 0.f;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = __builtin_amdgcn_exp2f(fmaf(st[qt][s][i], sc, -mu[qt]));
            sum += p;
            pf[qt][s * 4 + i] = (bf16)p;
          }
        l[qt] += sum;
      }
      const char *Vb = smem + (t % NBUF) * STAGE + KV_B;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int piece = dt * 2 + vpiece;
        const att_s4 lo = lds_read_tr16(Vb + vr * RB + ((piece ^ vsw0) << 4) + vbyte);
        const att_s4 hi = lds_read_tr16(Vb + (vr + 4) * RB + ((piece ^ vsw1) << 4) + vbyte);
        const frag vf = __builtin_bit_cast(frag, (att_s8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) o[qt][dt] = Mfma<bf16>::mma(vf, pf[qt], o[qt][dt]);
      }
    };
    // new column maxima from tile t's scores; rescales the running sums and outputs (one
    // wave-uniform branch, taken only when some column's maximum grew)
    auto new_max = [&](f32x4(&st)[2][2], float(&mu)[2]) {
      bool grow = false;
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        float mx = fmaxf(fmaxf(st[qt][0][0], st[qt][0][1]), fmaxf(st[qt][0][2], st[qt][0][3]));
        mx = fmaxf(mx, fmaxf(fmaxf(st[qt][1][0], st[qt][1][1]), fmaxf(st[qt][1][2], st[qt][1][3])));
        mx = max_xor32(max_xor16(mx)) * sc;
        const float m_new = fmaxf(m[qt], mx);
        mu[qt] = m_new == -INFINITY ? 0.f : m_new;
        grow |= m_new > m[qt];
      }
      if (__ballot(grow) != 0) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          const float alpha = __builtin_amdgcn_exp2f(m[qt] - mu[qt]);
          l[qt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[qt][dt] *= alpha;
        }
      }
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) m[qt] = fmaxf(m[qt], mu[qt]);
    };

    // Software pipeline: iteration t multiplies Q K^T of tile t+1 in the same basic block as the
    // exponentials and P V of tile t, so a wave's MFMAs overlap its own vector work.  Every tile
    // but the last is full (no masking, keys in both halves); the last one takes the general
    // path.  The row sums stay per lane (each lane sums its own keys; the maximum, and so every
    // rescale, is common to the column) and are reduced once at the end.
    f32x4 st_next[2][2];
    scores(0, st_next);  // a half without keys computes values that are never used
    for (int t = 0; t < nt - 1; ++t) {
      vm_wait_upto12(min(NBUF - 3, nt - 2 - t) * LPW);  // stage t+1 of this wave has landed
      wg_barrier();  // ... of every wave; stage t-1 is fully read
      if (t + NBUF - 1 < nt) issue(t + NBUF - 1);
      f32x4 st[2][2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int s = 0; s < 2; ++s) st[qt][s] = st_next[qt][s];
      float mu[2];
      new_max(st, mu);
      scores(t + 1, st_next);
      exp_pv(t, st, mu);
    }
    {
      const int t = nt - 1;
      vm_wait<0>();
      wg_barrier();
      const int kt0 = k_begin + t * TK + kh * 32;
      if (kt0 < k_end) {  // wave-uniform
        if (kt0 + 32 > k_end) {
#pragma unroll
          for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (kt0 + g * 8 + 4 * s + i >= k_end) st_next[qt][s][i] = -INFINITY;
        }
        float mu[2];
        new_max(st_next, mu);
        exp_pv(t, st_next, mu);
      }
    }
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) l[qt] = sum_xor32(sum_xor16(l[qt]));
  }
  __syncthreads();  // every copy has landed and every stage read is done: the LDS is free
  attn_finish<bf16, D>(a, smem, m, l, o, wave, lane, b, h, r0, nq, grp, chunk, nch);
}

// Merge the key chunks of every query slot (a separate launch: the kernel boundary makes the
// partial results visible, with no device-scope fence inside a kernel):
//   O = sum_c 2^(m_c - M) l_c O_c / sum_c 2^(m_c - M) l_c, summed in chunk order.
// One workgroup per (sample, KV head, query block, 16 slots); thread = one 16-byte vector of one
// slot's output, computing its slot's chunk weights itself (the 16 threads of a slot read the
// same statistics), every load issued before the first is used.
template <typename T, int D, int G, int NT>
__global__ __launch_bounds__(NT) void attn_combine_kernel(AttnArgs a) {
  typedef Mfma<T> MF;
  constexpr int EPL = MF::EPL, RPH = ATT_SLOTS / G, MAXC = 16;
  constexpr int VPRW = D / EPL;        // vectors per slot row
  constexpr int SPW = NT / VPRW;       // slots per workgroup
  const int tid = threadIdx.x;
  const int bk = blockIdx.x, qb = blockIdx.y, nqb = gridDim.y;
  const int b = bk / a.Hkv, kvh = bk - b * a.Hkv;
  // action queries: S rows, no wait for the prefix length; chunks past a sample's keys carry
  // weight 0, so every one of the n_chunks is merged
  const int nq = a.suffix ? a.S : max(0, min(a.lens[b], a.kp_rows));
  const int nch = a.n_chunks;
  const int slot = blockIdx.z * SPW + tid / VPRW, cv = tid % VPRW;
  const int srow = qb * RPH + slot % RPH;
  if (qb * RPH >= nq) return;
  const int HD = a.Hq * D;
  const size_t grp = (size_t)bk * nqb + qb;
  const T *part_o = (const T *)a.part;
  const float *part_ml = (const float *)((const char *)a.part +
                                         ((part_o_elems(a.B, a.Hkv, nqb, a.n_chunks, D) * sizeof(T) + 255) & ~(size_t)255));
  const float *pml = part_ml + grp * a.n_chunks * ATT_SLOTS * 2;
  float2 ml[MAXC];
  typename MF::frag pv[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {  // unconditional loads (clamped chunk) stay in flight together
    const int cc = min(c, nch - 1);
    ml[c] = *reinterpret_cast<const float2 *>(&pml[(cc * ATT_SLOTS + slot) * 2]);
    pv[c] = load_frag<T>(part_o + ((grp * a.n_chunks + cc) * ATT_SLOTS + slot) * D + cv * EPL);
  }
  float M = -INFINITY;
#pragma unroll
  for (int c = 0; c < MAXC; ++c)
    if (c < nch) M = fmaxf(M, ml[c].x);
  float w[MAXC], L = 0.f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    w[c] = c < nch && ml[c].y > 0.f ? __builtin_amdgcn_exp2f(ml[c].x - M) * ml[c].y : 0.f;
    L += w[c];
  }
  const float invL = 1.0f / L;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float t = w[c] * to_f32(pv[c][e]);
      acc[e] += w[c] > 0.f ? t : 0.f;  // a zero-weight chunk's output was never written
    }
  if (srow >= nq) return;
  const int hh = kvh * G + slot / RPH;
  typename MF::frag o8;
#pragma unroll
  for (int e = 0; e < EPL; ++e) o8[e] = from_f32<T>(acc[e] * invL);
  *reinterpret_cast<typename MF::frag *>((T *)a.out + (size_t)(b * a.q_rows_per_b + srow) * HD + hh * D + cv * EPL) = o8;
}

template <typename T, int D, int G> static void attn_t(const AttnArgs &a, hipStream_t s) {
  const int q_rows = a.suffix ? a.S : a.kp_rows;
  const int nqb = attn_qblocks(q_rows, a.Hq, a.Hkv);
  // (sample, KV head) varies fastest: consecutive workgroups go to consecutive XCDs, so all key
  // chunks of one KV head share an XCD and its L2 holds their partial results for the merge.
  dim3 grid(a.B * a.Hkv, nqb, a.n_chunks);
  if constexpr (std::is_same<T, bf16>::value && D == 128)
    hipLaunchKernelGGL((attn_dma_kernel<G, 4>), grid, dim3(ATT_THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((attn_kernel<T, D, G>), grid, dim3(ATT_THREADS), 0, s, a);
  if (a.n_chunks > 1) {
    // 256 threads per workgroup, or 64 when that leaves fewer than 256 workgroups (batch 1: the
    // merge is a latency chain, so more, smaller workgroups keep more loads in flight per CU)
    constexpr int VPRW = D / Mfma<T>::EPL;
    if ((size_t)a.B * a.Hkv * nqb * ATT_SLOTS * VPRW / 256 < 256)
      hipLaunchKernelGGL((attn_combine_kernel<T, D, G, 64>), dim3(a.B * a.Hkv, nqb, ATT_SLOTS * VPRW / 64), dim3(64), 0, s,
                         a);
    else
      hipLaunchKernelGGL((attn_combine_kernel<T, D, G, 256>), dim3(a.B * a.Hkv, nqb, ATT_SLOTS * VPRW / 256), dim3(256), 0,
                         s, a);
  }
}

template <typename T, int D> static void attn_g(const AttnArgs &a, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
    case 1: attn_t<T, D, 1>(a, s); break;
    case 2: attn_t<T, D, 2>(a, s); break;
    default: attn_t<T, D, 4>(a, s); break;
  }
}
template <typename T> static void attn_d(const AttnArgs &a, hipStream_t s) {
  switch (a.D) {
    case 32: attn_g<T, 32>(a, s); break;
    case 64: attn_g<T, 64>(a, s); break;
    default: attn_g<T, 128>(a, s); break;
  }
}
void launch_attention(Dt dt, const AttnArgs &a, hipStream_t s) {
  if (dt == DT_BF16) attn_d<bf16>(a, s); else attn_d<float>(a, s);
}

}  // namespace dm

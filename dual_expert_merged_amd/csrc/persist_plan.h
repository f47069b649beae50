// Work split of the single-launch batch-1 suffix denoise (persist.hip), as plain integer maps
// that the host and the device share: which weight rows and which cached keys a workgroup
// copies into its LDS, and where each copied 16-byte piece comes from.  Pure integer code with
// no HIP types, so the address maps can also be checked by an ordinary C++ compiler on the host.
//
// The 256 workgroups form 8 groups of 32 (group x = block % 8, the XCD the hardware places the
// block on; placement only affects speed).  Group x owns KV head x (its two query heads, its keys
// and values), 1/8 of the FFN columns, and a full copy of the residual stream; workgroup i of the
// group owns 32 residual columns.  Per layer, workgroup (x, i) keeps in LDS:
//   QKV : 16 rows of the fused Q/K/V weight (8 RoPE pairs of one query or key head of group x,
//         or 16 dims of its value head), all 1024 inputs                       32 KB
//   KV  : keys i*Pc .. i*Pc+Pc-1 of head x's cached prefix (K and V rows)      <= 16 KB
//   O   : O-projection rows 32i .. 32i+31 over the 256 inputs of group x's query heads   16 KB
//   GU  : gate and up rows of FFN columns 384x + 12i .. +11, all 1024 inputs    48 KB
//   D   : down-projection rows 32i .. 32i+31 over FFN inputs 384x .. 384x+383     24 KB
#pragma once

#ifdef __HIPCC__
#define PK_HD __host__ __device__ __forceinline__
#else
#define PK_HD inline
#endif

namespace dm {
namespace pk {

constexpr int NX = 8;             // groups = KV heads
constexpr int NG = 32;            // workgroups per group
constexpr int NWG = NX * NG;      // 256: one per CU
constexpr int H = 1024, F = 3072, HQ = 16, HKV = 8, D = 128;
constexpr int QKV_ROWS = (HQ + 2 * HKV) * D;  // 4096
constexpr int GW = 4 * D;         // per-group Q/K/V columns: two query heads, one key head, one value head
constexpr int HC = H / NG;        // 32 residual columns per workgroup
constexpr int FG = F / NX;        // 384 FFN columns per group
constexpr int FC = FG / NG;       // 12 FFN columns per workgroup
constexpr int SMAX = 64;          // action tokens per chunk
constexpr int AMAX = 32;          // action dim
constexpr int KROWS = 32;         // key rows per workgroup: prefix chunk + action keys
constexpr int PC_MAX = 30;        // prefix keys per workgroup (P_cap <= 960)
constexpr int SC_MAX = 2;         // action keys per workgroup (S <= 64)
constexpr int LMAX = 28;          // layers (norm gains kept in LDS)
constexpr int NCW = 8;            // compute waves
constexpr int NDW = 4;            // copy (DMA) waves
constexpr int THREADS = (NCW + NDW) * 64;

// LDS segments, in copy order within a layer.  A weight segment of R rows and K inputs is stored
// k-step-major: [K/64][R][128 bytes], the 16-byte chunk c of row r at position c ^ (r & 7).
enum Seg { SEG_QKV = 0, SEG_KV = 1, SEG_O = 2, SEG_GU = 3, SEG_D = 4, NSEG = 5 };
constexpr int SEG_ROWS[NSEG] = {16, 0, 32, 24, 32};
constexpr int SEG_K[NSEG] = {H, 0, 2 * D, H, FG};
// 1 KB lines (one global_load_lds_dwordx4 of a wave) per segment
constexpr int SEG_LINES[NSEG] = {16 * 16 / 8, 2 * KROWS / 4, 4 * 32 / 8, 16 * 24 / 8, 6 * 32 / 8};
constexpr int SEG_BYTES[NSEG] = {SEG_LINES[0] * 1024, SEG_LINES[1] * 1024, SEG_LINES[2] * 1024, SEG_LINES[3] * 1024,
                                 SEG_LINES[4] * 1024};
static_assert(SEG_LINES[0] % NDW == 0 && SEG_LINES[1] % NDW == 0 && SEG_LINES[2] % NDW == 0 &&
                  SEG_LINES[3] % NDW == 0 && SEG_LINES[4] % NDW == 0,
              "every segment splits evenly over the copy waves");

// The phases of a layer-step, and the one that reads each segment.
enum Phase { PH_QKV = 0, PH_ATT, PH_MRG, PH_OPJ, PH_RDO, PH_GU, PH_DN, PH_RDD, NPH };
constexpr int SEG_READER[NSEG] = {PH_QKV, PH_ATT, PH_OPJ, PH_GU, PH_DN};

// Copy schedule of a copy wave, in 1 KB lines of its share of each segment (SEG_LINES / NDW
// lines).  At the start of phase ph of layer-step ls the wave issues up to two pieces
// {segment, layer-step (0: ls, 1: ls + 1), first line, end line} (seg < 0: none), then waits
// until at most COPY_WAIT[ph] of its copies are in flight (-1: no wait).  Copies complete in
// issue order, so a wait count is the number of this wave's copies issued after the last line
// of the segment the phase reads.  A segment is refilled for ls + 1 only after its reader phase
// of ls, in pieces spread over the following phases, so that no phase starts behind a large
// burst of copies.  Layer-step 0's segments are all copied before the first phase (the pieces
// "of ls" in layer-step 0 then repeat identical bytes), and in the last layer-step nothing of a
// next one is issued and every wait is for all copies.
struct CopyPiece {
  int seg, next, u0, u1;
};
constexpr int COPY_PIECES = 2;
constexpr CopyPiece COPY_PLAN[NPH][COPY_PIECES] = {
    {{SEG_GU, 0, 10, 12}, {SEG_D, 0, 2, 4}},  // QKV
    {{SEG_QKV, 1, 0, 4}, {-1, 0, 0, 0}},      // ATT
    {{SEG_QKV, 1, 4, 8}, {-1, 0, 0, 0}},      // MRG
    {{SEG_KV, 1, 0, 4}, {-1, 0, 0, 0}},       // OPJ
    {{SEG_O, 1, 0, 4}, {-1, 0, 0, 0}},        // RDO
    {{SEG_D, 0, 4, 6}, {-1, 0, 0, 0}},        // GU
    {{SEG_GU, 1, 0, 6}, {-1, 0, 0, 0}},       // DN
    {{SEG_GU, 1, 6, 10}, {SEG_D, 1, 0, 2}},   // RDD
};
constexpr int COPY_WAIT[NPH] = {26, 26, -1, 30, -1, 20, 6, -1};

// Chunk permutation of the 256-byte key / value rows: chunk c of row r sits at position
// c ^ kv_swz(r), which keeps the score-tile reads and the transposing value reads free of bank
// conflicts.
PK_HD int kv_swz(int r) { return ((r & 3) << 1) | (r & 8) | (((r >> 4) ^ (r >> 2)) & 1); }

// Global row of the fused Q/K/V weight held in LDS row r (0..15) by workgroup i of group x, and
// the matching column of the group's Q/K/V buffer [S][GW] (query head 2x, query head 2x+1, key
// head x, value head x, 128 columns each).  Workgroups 0..23 take 8 rotary pairs (dims d and
// d + 64 in rows r and r + 8) of one query or key head; 24..31 take 16 dims of the value head.
PK_HD int qkv_local_col(int i, int r) {
  if (i < 24) {
    const int sec = i >> 3, p = i & 7;
    const int dim = r < 8 ? 8 * p + r : 64 + 8 * p + (r - 8);
    return sec * D + dim;
  }
  return 3 * D + 16 * (i - 24) + r;
}
PK_HD int qkv_global_row(int x, int i, int r) {
  const int c = qkv_local_col(i, r), sec = c / D, dim = c % D;
  if (sec < 2) return (2 * x + sec) * D + dim;         // query heads 2x, 2x+1
  if (sec == 2) return HQ * D + x * D + dim;           // key head x
  return (HQ + HKV) * D + x * D + dim;                 // value head x
}

// Source of one 16-byte DMA piece of a weight segment: line `line` of the segment, lane `lane`
// (0..63).  Returns the element offset into the layer's weight matrix (row-major [rows][K_full])
// and sets *which to 0 (the segment's matrix) or 1 (the up-projection for GU rows >= 12).
PK_HD long weight_piece(int seg, int x, int i, int line, int lane, int *which) {
  const int R = SEG_ROWS[seg];
  const int kstep = line / (R / 8), rb = line % (R / 8);
  const int row = rb * 8 + (lane >> 3), pos = lane & 7;
  const int chunk = pos ^ (row & 7);
  const int k = kstep * 64 + chunk * 8;
  *which = 0;
  switch (seg) {
    case SEG_QKV: return (long)qkv_global_row(x, i, row) * H + k;
    case SEG_O: return (long)(HC * i + row) * (HQ * D) + 2 * D * x + k;
    case SEG_GU:
      if (row >= FC) *which = 1;
      return (long)(FG * x + FC * i + (row % FC)) * H + k;
    default: return (long)(HC * i + row) * F + FG * x + k;  // SEG_D
  }
}

// Source of one 16-byte DMA piece of the KV segment: element offset into the head's cache block
// [P_cap][D] (K for lines 0..7, V for lines 8..15) of the prefix key i*Pc + r, clamped into the
// cache (rows past the chunk are copied but never used).  LDS row = line * 4 + lane / 16
// (K rows 0..31, then V rows 0..31).
PK_HD long kv_piece(int i, int Pc, int P, int line, int lane, int *is_v) {
  const int lrow = line * 4 + (lane >> 4), pos = lane & 15;
  const int r = lrow & (KROWS - 1);
  *is_v = lrow >= KROWS;
  int key = i * Pc + r;
  const int last = P > 0 ? P - 1 : 0;
  if (key > last) key = last;
  const int chunk = pos ^ kv_swz(r);
  return (long)key * D + chunk * 8;
}

// Prefix keys per workgroup for a prefix of P tokens, and action keys per workgroup.
PK_HD int prefix_chunk(int P) { return (P + NG - 1) / NG; }
PK_HD int action_chunk(int S) { return (S + NG - 1) / NG; }

}  // namespace pk
}  // namespace dm

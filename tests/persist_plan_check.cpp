// Host-side check of the single-launch denoise's copy maps (persist_plan.h), built with g++ by
// tests/test_persist_plan.py: every 16-byte piece a workgroup copies lies inside its matrix or
// cache block, every LDS position of a segment is filled exactly once, and the workgroups of a
// group together copy exactly the weight rows (and key rows) the group owns; the copy schedule
// (COPY_PLAN / COPY_WAIT) delivers every segment before it is read and never overwrites one
// while it is read.
#include <algorithm>
#include <cstdio>
#include <set>
#include <vector>

#include "persist_plan.h"

using namespace dm::pk;

static int fails = 0;
#define CHECK(c, ...)                 \
  do {                                \
    if (!(c)) {                       \
      if (fails < 20) printf(__VA_ARGS__); \
      ++fails;                        \
    }                                 \
  } while (0)

int main() {
  const long full_rows[NSEG] = {QKV_ROWS, 0, H, F, H};
  const long full_k[NSEG] = {H, 0, HQ * D, H, F};
  for (int x = 0; x < NX; ++x) {
    std::set<long> qkv_rows, o_rows, gate_rows, up_rows, d_rows;
    for (int i = 0; i < NG; ++i) {
      for (int seg : {SEG_QKV, SEG_O, SEG_GU, SEG_D}) {
        const int R = SEG_ROWS[seg], K = SEG_K[seg];
        std::vector<int> filled(R * K / 8, 0);  // (row, 8-element chunk) of the segment
        for (int line = 0; line < SEG_LINES[seg]; ++line)
          for (int lane = 0; lane < 64; ++lane) {
            int which = 0;
            const long e = weight_piece(seg, x, i, line, lane, &which);
            CHECK(e >= 0 && e + 8 <= full_rows[seg] * full_k[seg], "seg %d x %d i %d line %d lane %d: offset %ld out of range\n",
                  seg, x, i, line, lane, e);
            CHECK(e % 8 == 0, "seg %d: offset %ld not 16-byte aligned\n", seg, e);
            const long grow = e / full_k[seg], gk = e % full_k[seg];
            // LDS position of this lane's piece and the (row, chunk) the kernel reads there
            const int byte = line * 1024 + lane * 16;
            const int kstep = byte / (R * 128), row = (byte % (R * 128)) / 128, pos = (byte % 128) / 16;
            const int chunk = pos ^ (row & 7);
            CHECK(kstep * 64 + chunk * 8 < K, "seg %d: LDS position past K\n", seg);
            filled[row * (K / 8) + kstep * 8 + chunk] += 1;
            // the global piece must be that (row, k) of the workgroup's rows
            long want_row;
            int want_which = 0;
            long kofs = 0;
            if (seg == SEG_QKV) want_row = qkv_global_row(x, i, row);
            else if (seg == SEG_O) want_row = HC * i + row, kofs = 2 * D * x;
            else if (seg == SEG_GU) want_row = FG * x + FC * i + row % FC, want_which = row >= FC;
            else want_row = HC * i + row, kofs = FG * x;
            CHECK(grow == want_row && gk == kofs + kstep * 64 + chunk * 8 && which == want_which,
                  "seg %d x %d i %d line %d lane %d: row %ld k %ld, expected row %ld k %ld\n", seg, x, i, line, lane, grow,
                  gk, want_row, kofs + kstep * 64 + chunk * 8);
            if (seg == SEG_QKV) qkv_rows.insert(grow);
            if (seg == SEG_O) o_rows.insert(grow);
            if (seg == SEG_GU) (which ? up_rows : gate_rows).insert(grow);
            if (seg == SEG_D) d_rows.insert(grow);
          }
        for (size_t c = 0; c < filled.size(); ++c)
          CHECK(filled[c] == 1, "seg %d x %d i %d: LDS chunk %zu filled %d times\n", seg, x, i, c, filled[c]);
      }
      // the output columns of the fused Q/K/V rows: 4 consecutive rows -> 4 consecutive columns
      for (int r0 = 0; r0 < 16; r0 += 4)
        for (int j = 1; j < 4; ++j)
          CHECK(qkv_local_col(i, r0 + j) == qkv_local_col(i, r0) + j, "qkv columns of i %d rows %d.. not consecutive\n", i, r0);
      // rotary pairs: row r and r + 8 hold dims d and d + 64 of one query / key head
      if (i < 24)
        for (int r = 0; r < 8; ++r)
          CHECK(qkv_local_col(i, r + 8) == qkv_local_col(i, r) + 64, "pair rows %d of i %d\n", r, i);
    }
    // the group copies exactly its own rows
    std::set<long> want_qkv;
    for (int d = 0; d < D; ++d) {
      want_qkv.insert((2 * x) * D + d);
      want_qkv.insert((2 * x + 1) * D + d);
      want_qkv.insert(HQ * D + x * D + d);
      want_qkv.insert((HQ + HKV) * D + x * D + d);
    }
    CHECK(qkv_rows == want_qkv, "group %d: Q/K/V rows differ from its heads' rows\n", x);
    CHECK((long)o_rows.size() == H && *o_rows.begin() == 0 && *o_rows.rbegin() == H - 1, "group %d: O rows\n", x);
    CHECK((long)d_rows.size() == H && *d_rows.begin() == 0 && *d_rows.rbegin() == H - 1, "group %d: down rows\n", x);
    CHECK((long)gate_rows.size() == FG && *gate_rows.begin() == FG * x && *gate_rows.rbegin() == FG * x + FG - 1,
          "group %d: gate rows\n", x);
    CHECK(up_rows == gate_rows, "group %d: up rows differ from gate rows\n", x);
  }
  // keys: every prefix key of a head is copied by exactly one workgroup, at its row, inside the
  // cache block, for every prefix length the kernel accepts
  for (int P_cap : {1, 64, 816, 960})
    for (int P : {0, 1, 2, 31, 33, 100, 815, 816, 960}) {
      if (P > P_cap) continue;
      const int Pc = prefix_chunk(P);
      CHECK(Pc <= PC_MAX, "P %d: chunk %d too long\n", P, Pc);
      std::vector<int> seen(P > 0 ? P : 1, 0);
      for (int i = 0; i < NG; ++i) {
        const int nkp = std::max(0, std::min(Pc, P - i * Pc));
        for (int line = 0; line < SEG_LINES[SEG_KV]; ++line)
          for (int lane = 0; lane < 64; ++lane) {
            int is_v = 0;
            const long e = kv_piece(i, Pc, P, line, lane, &is_v);
            CHECK(e >= 0 && e + 8 <= (long)P_cap * D && e % 8 == 0, "kv P_cap %d P %d i %d line %d lane %d: %ld\n", P_cap,
                  P, i, line, lane, e);
            const int lrow = line * 4 + lane / 16, r = lrow % KROWS, pos = lane % 16;
            CHECK(is_v == (lrow >= KROWS), "kv: K/V half\n");
            const long key = e / D, chunk = (e % D) / 8;
            CHECK(chunk == (pos ^ kv_swz(r)), "kv: chunk position\n");
            if (r < nkp) {
              CHECK(key == (long)i * Pc + r, "kv: key of row %d\n", r);
              if (!is_v && pos == 0) seen[key] += 1;
            }
          }
      }
      for (int k = 0; k < P; ++k) CHECK(seen[k] == 1, "P %d: key %d copied %d times\n", P, k, seen[k]);
      const int Sc = action_chunk(SMAX);
      CHECK(Pc + Sc <= KROWS, "P %d: prefix + action keys exceed the key rows\n", P);
    }
  // The copy schedule, simulated per copy wave over whole chunks of 1..7 layer-steps: copies
  // complete in issue order and a wait retires the oldest until at most COPY_WAIT remain.  When a
  // phase reads a segment, every line must hold that layer-step's data with no copy of other data
  // still in flight to it; a refill for the next layer-step may only start after the segment's
  // reader phase; at most 63 copies are ever in flight (the counter's range).
  for (int T = 1; T <= 7; ++T) {
    struct Copy { int seg, u, ls; };
    std::vector<Copy> fifo;
    int holds[NSEG][16];
    for (auto &h : holds)
      for (int &v : h) v = -1;
    auto per = [](int seg) { return SEG_LINES[seg] / NDW; };
    auto retire_to = [&](int n) {
      while ((int)fifo.size() > n) {
        holds[fifo.front().seg][fifo.front().u] = fifo.front().ls;
        fifo.erase(fifo.begin());
      }
    };
    for (int seg : {SEG_QKV, SEG_KV, SEG_O, SEG_GU, SEG_D})
      for (int u = 0; u < per(seg); ++u) fifo.push_back({seg, u, 0});
    CHECK((int)fifo.size() <= 63, "start-up copies exceed the counter\n");
    for (int ls = 0; ls < T; ++ls) {
      const bool more = ls + 1 < T;
      for (int ph = 0; ph < NPH; ++ph) {
        for (int k = 0; k < COPY_PIECES; ++k) {
          const CopyPiece c = COPY_PLAN[ph][k];
          if (c.seg < 0 || (c.next && !more)) continue;
          CHECK(c.u0 >= 0 && c.u0 < c.u1 && c.u1 <= per(c.seg), "phase %d piece %d: line range\n", ph, k);
          if (c.next) CHECK(SEG_READER[c.seg] < ph, "phase %d refills segment %d before its reader\n", ph, c.seg);
          else CHECK(SEG_READER[c.seg] > ph, "phase %d copies segment %d of this layer-step after its reader\n", ph, c.seg);
          for (int u = c.u0; u < c.u1; ++u) fifo.push_back({c.seg, u, ls + c.next});
        }
        CHECK((int)fifo.size() <= 63, "T %d ls %d phase %d: %zu copies in flight\n", T, ls, ph, fifo.size());
        if (COPY_WAIT[ph] >= 0) retire_to(more ? COPY_WAIT[ph] : 0);
        for (int seg = 0; seg < NSEG; ++seg) {
          if (SEG_READER[seg] != ph) continue;
          for (int u = 0; u < per(seg); ++u) {
            CHECK(holds[seg][u] == ls, "T %d ls %d: segment %d line %d holds layer-step %d when read\n", T, ls, seg, u,
                  holds[seg][u]);
            for (const Copy &f : fifo)
              CHECK(!(f.seg == seg && f.u == u && f.ls != ls), "T %d ls %d: segment %d line %d overwritten while read\n",
                    T, ls, seg, u);
          }
        }
      }
    }
    retire_to(0);
  }
  // each segment is refilled exactly once per layer-step (and the total matches SEG_LINES)
  for (int seg = 0; seg < NSEG; ++seg) {
    std::vector<int> n(SEG_LINES[seg] / NDW, 0);
    for (int ph = 0; ph < NPH; ++ph)
      for (int k = 0; k < COPY_PIECES; ++k)
        if (COPY_PLAN[ph][k].seg == seg)
          for (int u = COPY_PLAN[ph][k].u0; u < COPY_PLAN[ph][k].u1; ++u) n[u] += 1;
    for (size_t u = 0; u < n.size(); ++u) CHECK(n[u] == 1, "segment %d line %zu copied %d times per layer-step\n", seg, u, n[u]);
  }
  // the swizzle is a permutation of the 16 chunk positions for every row
  for (int r = 0; r < KROWS; ++r) {
    std::set<int> p;
    for (int c = 0; c < 16; ++c) p.insert(c ^ kv_swz(r));
    CHECK(p.size() == 16, "kv_swz row %d\n", r);
  }
  printf(fails ? "FAILED %d checks\n" : "all copy maps consistent\n", fails);
  return fails ? 1 : 0;
}

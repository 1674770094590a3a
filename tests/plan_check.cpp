// Host-side checks of the launch plan (compiled with g++ by tests/test_plan.py).
#include <cstdio>
#include <cstdlib>
#include <set>
#include <tuple>
#include <vector>

#include "plan.h"

#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c);           \
      std::exit(1);                                                     \
    }                                                                   \
  } while (0)

static void check_plan(int B, int Hq, int Hkv, int Nq, int Nk, int causal, int qpw, int nw) {
  fa_plan_t p = fa_make_plan(B, Hq, Hkv, Nq, Nk, causal, qpw, nw);
  CHECK(p.hw >= 1 && nw % p.hw == 0 && p.G % p.hw == 0);
  CHECK(p.pos * p.hw == qpw * nw);
  // every (b, query head, query row) is covered by exactly one wave
  std::vector<int> cover((size_t)B * Hq * Nq, 0);
  std::set<std::tuple<int, int, int>> seen;
  long long last_work = -1;
  for (long long id = 0; id < p.nwg; ++id) {
    fa_work_t w = fa_decode(p, id);
    CHECK(w.b >= 0 && w.b < B && w.hkv >= 0 && w.hkv < Hkv);
    CHECK(w.qpos0 >= 0 && w.qpos0 < Nq && w.qpos0 % p.pos == 0);
    CHECK(seen.insert({w.b, w.hq0, w.qpos0}).second);  // bijection
    for (int wave = 0; wave < nw; ++wave) {
      int hq = w.hq0 + wave % p.hw;
      CHECK(hq / (Hq / Hkv) == w.hkv);                 // GQA: the head reads its own kv head
      int q0 = w.qpos0 + (wave / p.hw) * qpw;
      for (int i = q0; i < q0 + qpw && i < Nq; ++i) cover[((size_t)w.b * Hq + hq) * Nq + i]++;
    }
    // tile count: the last visible key of the workgroup's last row
    int nt = fa_num_kv_tiles(p, w.qpos0, 64);
    int qlast = w.qpos0 + p.pos - 1 < Nq - 1 ? w.qpos0 + p.pos - 1 : Nq - 1;
    int klast = causal ? (qlast + Nk - Nq < Nk - 1 ? qlast + Nk - Nq : Nk - 1) : Nk - 1;
    CHECK(nt == (klast < 0 ? 0 : klast / 64 + 1));
    if (nt > 0) CHECK(nt * 64 >= klast + 1 && (nt - 1) * 64 <= klast);
    (void)last_work;
  }
  CHECK((long long)seen.size() == p.nwg);
  for (int c : cover) CHECK(c == 1);
  // where the first two ids are the first two of the logical order, causal
  // workgroups of one group come heaviest first
  if (causal && (p.xcd == 0 || p.xcd == 8) && p.nqb > 1) {
    fa_work_t a = fa_decode(p, 0), b = fa_decode(p, 1);
    CHECK(a.qpos0 > b.qpos0);
  }
}

// Split plans: every (b, query head, query row, key tile) visible to the row
// is covered by exactly one (workgroup, tile in its range).
static void check_split(int B, int Hq, int Hkv, int Nq, int Nk, int causal, int nw, int tps) {
  fa_plan_t p = fa_split_plan(fa_make_plan(B, Hq, Hkv, Nq, Nk, causal, 32, nw), tps, 64);
  const int tiles = (Nk + 63) / 64;
  CHECK(p.nsplit >= 1 && p.tps >= 1 && (long long)p.nsplit * p.tps >= tiles && (long long)(p.nsplit - 1) * p.tps < tiles);
  std::vector<int> cover((size_t)B * Hq * Nq * tiles, 0);
  std::set<std::tuple<int, int, int, int>> seen;
  for (long long id = 0; id < p.nwg; ++id) {
    fa_work_t w = fa_decode(p, id);
    CHECK(w.split >= 0 && w.split < p.nsplit);
    CHECK(seen.insert({w.b, w.hq0, w.qpos0, w.split}).second);
    int nt = fa_num_kv_tiles(p, w.qpos0, 64), t0, t1;
    fa_split_tiles(p, w.split, nt, t0, t1);
    CHECK(0 <= t0 && t0 <= t1 && t1 <= nt);
    for (int wave = 0; wave < nw; ++wave) {
      int hq = w.hq0 + wave % p.hw;
      int q0 = w.qpos0 + (wave / p.hw) * 32;
      for (int i = q0; i < q0 + 32 && i < Nq; ++i) {
        int klast = causal ? (i + Nk - Nq < Nk - 1 ? i + Nk - Nq : Nk - 1) : Nk - 1;
        for (int t = t0; t < t1; ++t)
          if (t * 64 <= klast) cover[(((size_t)w.b * Hq + hq) * Nq + i) * tiles + t]++;
      }
    }
  }
  CHECK((long long)seen.size() == p.nwg);
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < Hq; ++h)
      for (int i = 0; i < Nq; ++i) {
        int klast = causal ? (i + Nk - Nq < Nk - 1 ? i + Nk - Nq : Nk - 1) : Nk - 1;
        for (int t = 0; t < tiles; ++t)
          CHECK(cover[(((size_t)b * Hq + h) * Nq + i) * tiles + t] == (klast >= 0 && t * 64 <= klast ? 1 : 0));
      }
  // the ranges of one query block are consecutive in the logical order
  if ((p.xcd == 0 || p.xcd == 8) && p.nsplit > 1) {
    fa_work_t a = fa_decode(p, 0), b = fa_decode(p, 1);
    CHECK(a.split == 0 && b.split == 1 && a.qpos0 == b.qpos0 && a.hq0 == b.hq0);
  }
}

// XCD remap of causal grids: the k XCDs that share a piece of the order hold
// whole runs (query or key blocks of one group) and the busiest XCD gets at
// most `slack` times the average work (key tiles, or query tiles for the
// backward's key blocks).
static void check_xcd_ways(long long nwg, long long run, int ways) {
  CHECK(ways == fa_xcd_ways(nwg, run, 1));
  if (ways == 0) return;
  CHECK(nwg % 8 == 0 && (ways == 8 || (ways * (nwg / 8)) % run == 0));
  for (int k = 1; k < ways; k *= 2) CHECK((k * (nwg / 8)) % run != 0);  // the smallest such pieces
  std::set<long long> seen;
  for (long long id = 0; id < nwg; ++id) CHECK(seen.insert(fa_xcd_order(id, nwg, ways)).second);
  CHECK(*seen.begin() == 0 && *seen.rbegin() == nwg - 1);
}
static void check_balance(const fa_plan_t& p, double slack) {
  CHECK(p.causal && p.xcd > 0);
  check_xcd_ways(p.nwg, (long long)p.nqb * p.nsplit, p.xcd);
  double load[8] = {0}, total = 0;
  for (long long id = 0; id < p.nwg; ++id) {
    const double t = fa_num_kv_tiles(p, fa_decode(p, id).qpos0, 64);
    load[id % 8] += t;
    total += t;
  }
  for (double l : load) CHECK(l <= slack * total / 8);
}
static void check_kv_balance(const fa_kvplan_t& p, double slack) {
  CHECK(p.causal && p.xcd > 0);
  check_xcd_ways(p.nwg, p.nkb, p.xcd);
  double load[8] = {0}, total = 0;
  for (long long id = 0; id < p.nwg; ++id) {
    int first, ntq;
    fa_kv_query_tiles(p, fa_kv_decode(p, id).k0, 64, first, ntq);
    load[id % 8] += ntq - first;
    total += ntq - first;
  }
  for (double l : load) CHECK(l <= slack * total / 8);
}

// Persistent grids of G workgroups: every work item is taken exactly once,
// by a workgroup on the XCD the hardware would have sent it to (id % 8), the
// rounds end for good once they run out, and with `slack` > 0 the busiest
// workgroup gets at most slack times the average key tiles.
static void check_persistent(const fa_plan_t& p, unsigned G, double slack) {
  std::vector<int> seen((size_t)p.nwg, 0);
  std::vector<double> load(G, 0.0);
  double total = 0;
  for (unsigned g = 0; g < G; ++g) {
    unsigned r = 0, last = 0;
    for (;; ++r) {
      const unsigned id = fa_persistent_item(G, p.nwg, g, r);
      if (id == ~0u) break;
      CHECK((long long)id < p.nwg && id % 8 == g % 8);
      CHECK(r == 0 || id > last);  // an XCD's ids in the hardware's order
      last = id;
      seen[id]++;
      const double t = fa_num_kv_tiles(p, fa_decode(p, id).qpos0, 64);
      load[g] += t;
      total += t;
    }
    for (unsigned k = 1; k < 4; ++k) CHECK(fa_persistent_item(G, p.nwg, g, r + k) == ~0u);
    if ((long long)G >= p.nwg) CHECK(r == ((long long)g < p.nwg ? 1u : 0u));
  }
  for (int v : seen) CHECK(v == 1);
  if (slack > 0)
    for (double l : load) CHECK(l <= slack * total / G);
}

// Backward key-block plans: every (b, kv head, key) is owned by exactly one
// wave, and every query row that sees one of a workgroup's keys lies in the
// query tiles the workgroup visits.
static void check_kvplan(int B, int Hq, int Hkv, int Nq, int Nk, int causal, int kpw, int nw) {
  fa_kvplan_t p = fa_make_kvplan(B, Hq, Hkv, Nq, Nk, causal, kpw, nw);
  CHECK(p.kpb == kpw * nw && (long long)p.nkb * p.kpb >= Nk && (long long)(p.nkb - 1) * p.kpb < Nk);
  std::vector<int> cover((size_t)B * Hkv * Nk, 0);
  std::set<std::tuple<int, int, int>> seen;
  for (long long id = 0; id < p.nwg; ++id) {
    fa_kvwork_t w = fa_kv_decode(p, id);
    CHECK(w.b >= 0 && w.b < B && w.hkv >= 0 && w.hkv < Hkv && w.k0 >= 0 && w.k0 < Nk && w.k0 % p.kpb == 0);
    CHECK(seen.insert({w.b, w.hkv, w.k0}).second);
    for (int j = w.k0; j < w.k0 + p.kpb && j < Nk; ++j) cover[((size_t)w.b * Hkv + w.hkv) * Nk + j]++;
    int first, ntq;
    fa_kv_query_tiles(p, w.k0, 64, first, ntq);
    CHECK(ntq == (Nq + 63) / 64 && 0 <= first && first <= ntq);
    for (int i = 0; i < Nq; ++i) {
      bool sees = !causal || w.k0 <= i + Nk - Nq;  // the block's first key is its most visible one
      if (sees) CHECK(i / 64 >= first);
    }
    if (first > 0) CHECK(causal && (first * 64 - 1) + Nk - Nq < w.k0);  // the skipped rows see none of the keys
  }
  CHECK((long long)seen.size() == p.nwg);
  for (int c : cover) CHECK(c == 1);
  if ((p.xcd == 0 || p.xcd == 8) && p.nkb > 1) CHECK(fa_kv_decode(p, 0).k0 == 0 && fa_kv_decode(p, 1).k0 == p.kpb);
}

// Key plans whose groups' query heads are split into parts: every
// (b, query head, key) is covered by exactly one workgroup, whose part holds
// the head, and the decode is a bijection onto (group, part, key block).
static void check_kvplan_split(int B, int Hq, int Hkv, int Nq, int Nk, int causal, int kpw, int nw, int parts) {
  fa_kvplan_t p = fa_split_kvplan_heads(fa_make_kvplan(B, Hq, Hkv, Nq, Nk, causal, kpw, nw), parts);
  CHECK(p.hsplit == parts && p.hps * parts == p.G && p.nwg == (long long)B * Hkv * p.nkb * parts);
  std::vector<int> cover((size_t)B * Hq * Nk, 0);
  std::set<std::tuple<int, int, int, int>> seen;
  for (long long id = 0; id < p.nwg; ++id) {
    fa_kvwork_t w = fa_kv_decode(p, id);
    CHECK(w.b >= 0 && w.b < B && w.hkv >= 0 && w.hkv < Hkv && w.hs >= 0 && w.hs < parts);
    CHECK(w.k0 >= 0 && w.k0 < Nk && w.k0 % p.kpb == 0);
    CHECK(seen.insert({w.b, w.hkv, w.hs, w.k0}).second);
    for (int hh = 0; hh < p.hps; ++hh) {
      const int hq = w.hkv * p.G + w.hs * p.hps + hh;
      CHECK(hq / p.G == w.hkv);
      for (int j = w.k0; j < w.k0 + p.kpb && j < Nk; ++j) cover[((size_t)w.b * Hq + hq) * Nk + j]++;
    }
  }
  for (int c : cover) CHECK(c == 1);
}

// Packed plans: every (b, query head, query row) is the column of exactly
// one (workgroup, wave, lane column), all heads of a workgroup read its kv
// head.
static void check_packed(int B, int Hq, int Hkv, int Nq, int Nk, int causal, int tps) {
  fa_plan_t p = fa_make_packed_plan(B, Hq, Hkv, Nq, Nk, causal);
  if (tps > 0) p = fa_split_plan(p, tps, 64);
  CHECK(p.pack * Nq <= 32 && p.pack * p.nw >= p.G && (p.nw & (p.nw - 1)) == 0 && p.nqb == 1 && p.nhg == 1);
  // the fewest waves: half as many would need more than 32 columns per wave
  if (p.nw > 1) CHECK((p.G + p.nw / 2 - 1) / (p.nw / 2) * Nq > 32);
  if (p.G * Nq <= 32) CHECK(p.nw == 1 && p.pack == p.G);
  const int tiles = (Nk + 63) / 64;
  std::vector<int> cover((size_t)B * Hq * Nq * tiles, 0);
  for (long long id = 0; id < p.nwg; ++id) {
    fa_work_t w = fa_decode(p, id);
    CHECK(w.qpos0 == 0 && w.hq0 == w.hkv * p.G);
    int nt = fa_num_kv_tiles(p, w.qpos0, 64), t0, t1;
    fa_split_tiles(p, w.split, nt, t0, t1);
    for (int wave = 0; wave < p.nw; ++wave)
    for (int col = 0; col < 32; ++col) {
      const int hh = col / Nq, head = wave * p.pack + hh;
      if (hh >= p.pack || head >= p.G) continue;  // an idle column
      const int hq = w.hq0 + head, i = col - hh * Nq;
      CHECK(hq / p.G == w.hkv && i < Nq);
      int klast = causal ? (i + Nk - Nq < Nk - 1 ? i + Nk - Nq : Nk - 1) : Nk - 1;
      for (int t = t0; t < t1; ++t)
        if (t * 64 <= klast) cover[(((size_t)w.b * Hq + hq) * Nq + i) * tiles + t]++;
    }
  }
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < Hq; ++h)
      for (int i = 0; i < Nq; ++i) {
        int klast = causal ? (i + Nk - Nq < Nk - 1 ? i + Nk - Nq : Nk - 1) : Nk - 1;
        for (int t = 0; t < tiles; ++t)
          CHECK(cover[(((size_t)b * Hq + h) * Nq + i) * tiles + t] == (klast >= 0 && t * 64 <= klast ? 1 : 0));
      }
}

// Shapes near the library's size limits (the coverage arrays of the checks
// above would not fit): sampled workgroup ids decode into range, tile counts
// follow the visibility rule and key ranges stay inside the tiles.  Built
// with the undefined-behaviour sanitizer, any signed overflow in the planning
// arithmetic fails here.
static unsigned long long lcg_state = 12345;
static long long sample_id(long long n) {
  lcg_state = lcg_state * 6364136223846793005ULL + 1442695040888963407ULL;
  return (long long)((lcg_state >> 17) % (unsigned long long)n);
}
static void check_large_plan(fa_plan_t p) {
  CHECK(p.nwg > 0 && p.nwg < (1LL << 31));
  const long long fixed[] = {0, 1, p.nwg / 2, p.nwg - 1};
  for (int s = 0; s < 2004; ++s) {
    const long long id = s < 4 ? fixed[s] : sample_id(p.nwg);
    fa_work_t w = fa_decode(p, id);
    CHECK(w.b >= 0 && w.b < p.B && w.hkv >= 0 && w.hkv < p.Hkv && w.hq0 >= 0 && w.hq0 < p.Hq);
    CHECK(w.hq0 / p.G == w.hkv && w.qpos0 >= 0 && w.qpos0 < p.Nq && w.split >= 0 && w.split < p.nsplit);
    const int nt = fa_num_kv_tiles(p, w.qpos0, 64);
    const long long rows = p.pack > 1 ? p.Nq : p.pos;
    const long long qlast = w.qpos0 + rows - 1 < p.Nq - 1 ? w.qpos0 + rows - 1 : p.Nq - 1;
    const long long kl = p.causal ? qlast + p.Nk - p.Nq : p.Nk - 1;
    const long long klast = kl < p.Nk - 1 ? kl : p.Nk - 1;
    CHECK(nt == (klast < 0 ? 0 : klast / 64 + 1));
    int t0, t1;
    fa_split_tiles(p, w.split, nt, t0, t1);
    CHECK(0 <= t0 && t0 <= t1 && (t1 <= nt || t0 == t1));
  }
}
static void check_large_kvplan(fa_kvplan_t p) {
  CHECK(p.nwg > 0 && p.nwg < (1LL << 31));
  for (int s = 0; s < 2004; ++s) {
    const long long id = s < 2 ? s * (p.nwg - 1) : sample_id(p.nwg);
    fa_kvwork_t w = fa_kv_decode(p, id);
    CHECK(w.b >= 0 && w.b < p.B && w.hkv >= 0 && w.hkv < p.Hkv && w.k0 >= 0 && w.k0 < p.Nk && w.k0 % p.kpb == 0);
    int first, ntq;
    fa_kv_query_tiles(p, w.k0, 64, first, ntq);
    CHECK(ntq == (p.Nq + 63) / 64 && 0 <= first && first <= ntq);
    if (first > 0) CHECK(p.causal && (long long)first * 64 - 1 + p.Nk - p.Nq < w.k0);
  }
}

int main() {
  for (int causal = 0; causal < 2; ++causal)
    for (int tps : {0, 1, 3, 100}) {
      check_packed(2, 8, 2, 1, 1000, causal, tps);     // decoding, GQA 4
      check_packed(1, 32, 1, 1, 300, causal, tps);     // MQA, 32 heads in one wave
      check_packed(3, 6, 2, 10, 200, causal, tps);     // 3 heads x 10 rows
      check_packed(1, 4, 2, 16, 70, causal, tps);      // 2 heads x 16 rows: all 32 columns
      check_packed(1, 8, 2, 7, 5, causal, tps);        // Nq > Nk: rows without keys
      check_packed(2, 64, 8, 8, 700, causal, tps);     // 8 heads x 8 rows: 2 waves
      check_packed(1, 24, 2, 10, 300, causal, tps);    // G = 12, 10 rows: 4 waves of 3 heads
      check_packed(1, 16, 1, 16, 129, causal, tps);    // G = 16, 16 rows: 8 waves of 2 heads
      check_packed(3, 12, 2, 5, 200, causal, tps);     // G = 6, 5 rows: 1 wave
    }
  for (int causal = 0; causal < 2; ++causal)
    for (int nw : {1, 2, 4})
      for (int kpw : {32, 64}) {
        check_kvplan(2, 32, 8, 8192, 8192, causal, kpw, nw);
        check_kvplan(1, 6, 2, 257, 300, causal, kpw, nw);
        check_kvplan(2, 4, 1, 1000, 70, causal, kpw, nw);
        check_kvplan(1, 2, 2, 150, 40, causal, kpw, nw);
        check_kvplan(1, 3, 3, 40, 150, causal, kpw, nw);
        check_kvplan(3, 5, 5, 1, 100, causal, kpw, nw);
      }
  for (int causal = 0; causal < 2; ++causal)
    for (int nw : {1, 2, 8}) {
      check_kvplan_split(2, 16, 1, 300, 700, causal, 32, nw, 4);   // MQA, 4 parts of 4 heads
      check_kvplan_split(1, 12, 2, 100, 333, causal, 64, nw, 3);   // G = 6 in 3 parts
      check_kvplan_split(3, 8, 8, 64, 100, causal, 32, nw, 1);     // G = 1: one part
      check_kvplan_split(1, 32, 2, 50, 260, causal, 32, nw, 16);   // one head per part
    }
  for (int causal = 0; causal < 2; ++causal)
    for (int tps : {1, 2, 3, 7, 100}) {
      check_split(2, 8, 2, 1, 1000, causal, 4, tps);    // decoding: one query, GQA 4
      check_split(1, 4, 4, 3, 513, causal, 1, tps);     // three queries
      check_split(1, 6, 2, 70, 300, causal, 2, tps);    // several query blocks
      check_split(1, 2, 2, 150, 40, causal, 1, tps);    // Nq > Nk
    }

  for (int causal = 0; causal < 2; ++causal)
    for (int nw : {1, 2, 4, 8})
      for (int qpw : {32, 64}) {
        check_plan(2, 32, 8, 8192, 8192, causal, qpw, nw);
        check_plan(8, 12, 12, 1024, 1024, causal, qpw, nw);
        check_plan(1, 6, 2, 257, 257, causal, qpw, nw);
        check_plan(2, 4, 2, 200, 333, causal, qpw, nw);
        check_plan(1, 8, 1, 130, 130, causal, qpw, nw);
        check_plan(1, 3, 3, 1, 77, causal, qpw, nw);
        check_plan(1, 2, 2, 150, 40, causal, qpw, nw);
        check_plan(3, 5, 5, 100, 100, causal, qpw, nw);
      }
  // XCD remap: the ids that land on one XCD (id % 8) form one contiguous block of the logical order
  fa_plan_t p = fa_make_plan(2, 32, 8, 8192, 8192, 1, 64, 4);
  CHECK(p.xcd == 1 && p.nwg == 2048);
  for (int x = 0; x < 8; ++x) {
    std::set<int> groups;
    for (long long id = x; id < p.nwg; id += 8) {
      fa_work_t w = fa_decode(p, id);
      groups.insert(w.b * p.Hkv + w.hkv);
    }
    CHECK(groups.size() == 2);  // 16 (b, kv head) groups over 8 XCDs
  }
  // the first ids of an XCD get the heaviest (last) query block
  CHECK(fa_decode(p, 0).qpos0 == 8192 - 64 && fa_decode(p, 8).qpos0 == 8192 - 128);
  // causal grids whose groups span several XCDs: the blocks of a group
  // alternate over them (k = 2, 4, 8), each XCD within 1 % of the average
  // work (one eighth holding part of a group had up to 1.9x)
  for (int causal = 0; causal < 2; ++causal) {
    check_plan(1, 16, 4, 32768, 32768, causal, 32, 8);   // 4 groups of 512 blocks: k = 2
    check_plan(1, 2, 2, 8192, 8192, causal, 32, 8);      // 2 groups of 32 blocks: k = 4
    check_plan(1, 8, 1, 32768, 32768, causal, 32, 8);    // MQA, one group of 1024 blocks: k = 8
    check_plan(1, 12, 12, 8192, 8192, causal, 32, 8);    // 12 groups of 32 blocks: k = 2
    check_kvplan(1, 4, 1, 32768, 32768, causal, 32, 4);  // one key group: k = 8
    check_kvplan(1, 6, 2, 8192, 8192, causal, 64, 4);    // 2 groups of 32 key blocks: k = 4
  }
  CHECK(fa_make_plan(1, 16, 4, 32768, 32768, 1, 32, 8).xcd == 2);
  CHECK(fa_make_plan(1, 2, 2, 8192, 8192, 1, 32, 8).xcd == 4);
  CHECK(fa_make_plan(1, 8, 1, 32768, 32768, 1, 32, 8).xcd == 8);
  CHECK(fa_make_plan(1, 16, 4, 32768, 32768, 0, 32, 8).xcd == 1);   // even work: contiguous eighths
  CHECK(fa_make_plan(2, 32, 8, 8192, 8192, 1, 32, 8).xcd == 1);     // 2 whole groups per XCD
  check_balance(fa_make_plan(1, 16, 4, 32768, 32768, 1, 32, 8), 1.01);
  check_balance(fa_make_plan(1, 8, 1, 32768, 32768, 1, 32, 8), 1.01);
  check_balance(fa_make_plan(1, 12, 12, 8192, 8192, 1, 32, 8), 1.01);
  check_balance(fa_make_plan(1, 2, 2, 8192, 8192, 1, 32, 8), 1.01);
  check_balance(fa_make_plan(2, 32, 8, 8192, 8192, 1, 32, 8), 1.01);
  check_balance(fa_split_plan(fa_make_plan(1, 4, 1, 2048, 2048, 1, 32, 4), 4, 64), 1.01);
  check_kv_balance(fa_make_kvplan(1, 4, 1, 32768, 32768, 1, 32, 4), 1.01);
  check_kv_balance(fa_make_kvplan(1, 6, 2, 8192, 8192, 1, 64, 4), 1.01);
  check_kv_balance(fa_split_kvplan_heads(fa_make_kvplan(1, 8, 1, 16384, 16384, 1, 32, 4), 2), 1.01);
  check_kv_balance(fa_make_kvplan(2, 32, 8, 8192, 8192, 1, 32, 4), 1.01);
  for (long long nwg : {8LL, 24LL, 64LL, 3000LL, 8000LL})
    for (long long run : {1LL, 2LL, 3LL, 5LL, 64LL, 1000LL})
      check_xcd_ways(nwg, run, fa_xcd_ways(nwg, run, 1));
  // persistent grids of the 8-wave forward kernel (one workgroup per CU)
  for (int causal = 0; causal < 2; ++causal) {
    const fa_plan_t h = fa_make_plan(2, 32, 8, 8192, 8192, causal, 32, 8);  // 2048 items
    check_persistent(h, 256, causal ? 1.01 : 1.0);
    check_persistent(h, 248, 0);
    check_persistent(h, 304, 0);
    check_persistent(h, 8, 0);
    check_persistent(h, 4096, 0);                                            // more workgroups than items
    check_persistent(fa_make_plan(1, 36, 9, 7350, 7350, causal, 32, 8), 256, 0);  // 1035 items
    check_persistent(fa_make_plan(1, 16, 4, 32768, 32768, causal, 32, 8), 256, causal ? 1.01 : 1.0);
    check_persistent(fa_make_plan(1, 8, 1, 32768, 32768, causal, 32, 8), 256, causal ? 1.01 : 1.0);
    check_persistent(fa_make_plan(3, 8, 2, 500, 700, causal, 32, 8), 16, 0);
    check_persistent(fa_split_plan(fa_make_plan(2, 8, 2, 300, 3000, causal, 32, 8), 5, 64), 64, 0);
  }
  {
    // near the size limit: ids stay in range and every workgroup's rounds
    // add up to the grid
    const fa_plan_t big = fa_make_plan(64, 128, 8, 1 << 20, 1 << 20, 1, 32, 8);
    long long count = 0;
    for (unsigned g = 0; g < 256; ++g)
      for (unsigned r = 0;; ++r) {
        const unsigned id = fa_persistent_item(256, big.nwg, g, r);
        if (id == ~0u) break;
        CHECK((long long)id < big.nwg && id % 8 == g % 8);
        ++count;
      }
    CHECK(count == big.nwg);
  }
  // plan choice keeps >= 1024 workgroups when possible
  fa_plan_t c2 = fa_choose_plan(8, 12, 12, 1024, 1024, 1, 32, 1024, 8);
  CHECK(c2.nw == 2 && c2.nwg == 8 * 12 * 16);
  fa_plan_t c3 = fa_choose_plan(2, 32, 8, 8192, 8192, 1, 32, 1024, 8);
  CHECK(c3.nw == 8 && c3.hw == 4 && c3.pos == 64 && c3.nwg == 2048);
  for (int causal = 0; causal < 2; ++causal) {
    check_large_plan(fa_make_plan(64, 128, 8, 1 << 20, 1 << 20, causal, 32, 8));   // 33.5 M workgroups
    check_large_plan(fa_make_plan(1, 1, 1, 8000000, 8000000, causal, 32, 4));      // d = 64 key limit
    check_large_plan(fa_make_plan(2, 64, 64, 1000000, 3000000, causal, 32, 2));    // Nq < Nk
    check_large_plan(fa_split_plan(fa_make_plan(4, 16, 2, 7, 8000000, causal, 32, 8), 1, 64));
    check_large_plan(fa_split_plan(fa_make_packed_plan(64, 32, 8, 1, 8000000, causal), 5, 64));
    check_large_kvplan(fa_make_kvplan(64, 128, 8, 1 << 20, 1 << 20, causal, 32, 8));
    check_large_kvplan(fa_make_kvplan(1, 4, 1, 8000000, 3000000, causal, 64, 4));
    check_large_kvplan(fa_make_kvplan(2, 8, 8, 5, 8000000, causal, 32, 1));
  }
  // forward wave counts: the occupancy rule of fa_forward_plan
  CHECK(fa_forward_plan(2, 32, 8, 8192, 8192, 1, 128, 0, 32).nw == 8);    // 2048 workgroups of 8 waves
  CHECK(fa_forward_plan(4, 16, 16, 4096, 4096, 1, 128, 0, 32).nw == 4);   // causal: 1024 of 8 are too few
  CHECK(fa_forward_plan(4, 16, 16, 4096, 4096, 0, 128, 0, 32).nw == 8);   // not causal: 1024 suffice
  CHECK(fa_forward_plan(16, 16, 16, 512, 512, 1, 128, 0, 32).nw == 4);    // 8 waves would leave 512
  CHECK(fa_forward_plan(4, 8, 8, 1024, 1024, 0, 128, 0, 32).nw == 4);     // never fewer than 4 at d = 128
  CHECK(fa_forward_plan(1, 1, 1, 1, 77, 0, 128, 0, 32).nw == 4);
  CHECK(fa_forward_plan(4, 16, 16, 4096, 4096, 0, 256, 0, 32).nw == 4);   // d = 256: always 4
  CHECK(fa_forward_plan(1, 2, 2, 70, 70, 1, 256, 0, 32).nw == 4);
  CHECK(fa_forward_plan(8, 12, 12, 1024, 1024, 1, 64, 0, 32).nw == 4);    // 768 workgroups of 4 waves
  CHECK(fa_forward_plan(1, 12, 12, 4096, 4096, 1, 64, 0, 32).nw == 2);    // 384 would be too few
  CHECK(fa_forward_plan(4, 16, 16, 8192, 8192, 0, 128, 1, 32).nw == 4);   // fp8: up to 4
  CHECK(fa_forward_plan(2, 8, 8, 2048, 2048, 1, 128, 1, 32).nw == 1);     // fp8 d <= 128: 1024 one-wave workgroups
  CHECK(fa_forward_plan(1, 8, 8, 2048, 2048, 1, 256, 1, 32).nw == 2);     // fp8 d = 256: at least 2
  for (int d : {64, 128, 256})
    for (int fp8 = 0; fp8 < 2; ++fp8) {
      const fa_plan_t f = fa_forward_plan(3, 12, 4, 333, 500, 1, d, fp8, 32);
      CHECK(f.nw >= (fp8 && d <= 128 ? 1 : 2) && f.nw <= (d == 128 && !fp8 ? 8 : 4));
      check_plan(3, 12, 4, 333, 500, 1, 32, f.nw);
    }
  std::printf("plan checks passed\n");
  return 0;
}

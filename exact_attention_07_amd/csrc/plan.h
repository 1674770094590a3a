// plan.h -- launch planning for the fused attention forward kernels.
//
// Pure C++ (no HIP types), so the host-side tests can compile it with g++.
// The same decode runs on the GPU at the top of every workgroup.
//
// Work partitioning (the FlashAttention-2 change the pages describe on
// "FlashAttention-4震撼发布" and "FlashAttention (SV)", section
// "FlashAttention-2 (2023)": parallelise over query blocks as well as over
// batch and heads):
//   * one wave owns `qpw` consecutive query rows of one query head and keeps
//     them for the whole pass (the resident Q tile);
//   * a workgroup holds `nw` waves that share every K/V tile staged in LDS,
//     so all its waves read the same key/value head: it covers `hw` query
//     heads of one GQA group (hw divides both nw and Hq/Hkv) times
//     `pos` = qpw*nw/hw query positions;
//   * workgroups are numbered group-major (group = batch, kv head, head
//     subset) with the query blocks of a group consecutive; for causal
//     masking the heaviest query block (the last one) comes first;
//   * the hardware hands workgroup ids round-robin to the 8 XCDs of an
//     MI355X, each with its own L2.  When the count divides by 8 the id is
//     remapped so that XCD x runs the x-th contiguous eighth of that order,
//     which keeps the workgroups that read one K/V head on one L2.  Causal
//     work falls along a group's query blocks, so an eighth that holds part
//     of a group would get only its heavy or only its light blocks: then the
//     k XCDs (k = 2, 4 or 8) whose k eighths hold whole groups take the
//     blocks of those groups in turn (fa_xcd_ways);
//   * optionally the keys are split into `nsplit` ranges of `tps` tiles
//     (for grids too small to fill the chip, e.g. decoding with few query
//     rows): each workgroup then covers one range and writes a partial
//     result that a merge combines ("FlashAttention (SV)", section
//     "Online-beräkning av Softmax": block statistics combine exactly).  The
//     ranges of one query block are consecutive in the order;
//   * with few query rows (G * Nq <= 32) the G query heads of a GQA group
//     can share one wave (`pack` = G): its 32 query columns hold row c % Nq
//     of head c / Nq, so one pass over the group's K/V computes all of them
//     (decoding: one row per head would otherwise leave 31 of 32 columns
//     idle in every matrix product).
#ifndef FA_PLAN_H
#define FA_PLAN_H

#if defined(__HIPCC__)
#define FA_HD __host__ __device__
#else
#define FA_HD
#endif

struct fa_plan_t {
  int B, Hq, Hkv, Nq, Nk;
  int causal;
  int G;      // Hq / Hkv, query heads per key/value head
  int qpw;    // query rows per wave
  int nw;     // waves per workgroup
  int hw;     // query heads per workgroup
  int pos;    // query positions per workgroup
  int nqb;    // query blocks per head: ceil(Nq / pos)
  int nhg;    // head subsets per GQA group: G / hw
  int xcd;    // XCD remap of the workgroup ids (fa_xcd_ways; 0: none)
  int nsplit; // key ranges (1: no split)
  int tps;    // key tiles per range (nsplit > 1)
  int pack;   // query heads sharing one wave's columns (1: one head per wave)
  long long nwg;  // workgroups in the grid
};

// XCD remap of a grid of nwg workgroups whose logical order is made of runs
// of `run` workgroups (one group's query or key blocks), heaviest first
// within a run when `uneven` (causal).  0: no remap (nwg is not a multiple
// of 8); 1: XCD x runs the x-th contiguous eighth of the order; k = 2, 4, 8:
// the order is cut into 8 / k pieces of k eighths, the smallest such pieces
// that hold whole runs, and the k XCDs of a piece take its workgroups in
// turn, in a snake (XCD 0 .. k-1, then k-1 .. 0), so that over a run that
// gets lighter block by block none of them always draws the heaviest.
FA_HD inline int fa_xcd_ways(long long nwg, long long run, int uneven) {
  if (nwg % 8 != 0) return 0;
  if (!uneven) return 1;
  const long long c = nwg / 8;
  for (int k = 1; k < 8; k *= 2)
    if ((k * c) % run == 0) return k;
  return 8;
}

// Position in the logical order of workgroup id under XCD remap `ways`: the
// id's XCD x = id % 8 runs its (id / 8)-th workgroup.  Grids hold at most
// 2^31 - 1 workgroups (the launch checks refuse larger ones), so 32-bit
// arithmetic holds every position (cheaper on the GPU than 64-bit division).
FA_HD inline long long fa_xcd_order(long long id, long long nwg, int ways) {
  if (ways == 0) return id;
  const unsigned k = (unsigned)ways, c = (unsigned)(nwg / 8), i = (unsigned)id;
  const unsigned x = i % 8, u = i / 8, r = x % k;
  return (long long)((x / k) * k * c + u * k + ((u & 1) ? k - 1 - r : r));
}

// Largest of {nw, nw/2, ..., 1} that divides g (nw is a power of two).
FA_HD inline int fa_heads_per_wg(int g, int nw) {
  int hw = nw;
  while (hw > 1 && (g % hw) != 0) hw >>= 1;
  return hw;
}

FA_HD inline fa_plan_t fa_make_plan(int B, int Hq, int Hkv, int Nq, int Nk, int causal, int qpw, int nw) {
  fa_plan_t p;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Nq = Nq; p.Nk = Nk; p.causal = causal;
  p.G = Hq / Hkv;
  p.qpw = qpw;
  p.nw = nw;
  p.hw = fa_heads_per_wg(p.G, nw);
  p.pos = qpw * nw / p.hw;
  p.nqb = (Nq + p.pos - 1) / p.pos;
  p.nhg = p.G / p.hw;
  p.nsplit = 1;
  p.tps = 0;
  p.pack = 1;
  p.nwg = (long long)B * Hkv * p.nhg * p.nqb;
  p.xcd = fa_xcd_ways(p.nwg, p.nqb, causal);
  return p;
}

// Waves of a packed workgroup: the fewest (a power of two) whose query
// columns hold all G heads' Nq rows, ceil(G / waves) heads per wave.
FA_HD inline int fa_packed_waves(int G, int Nq) {
  int nw = 1;
  while ((long long)((G + nw - 1) / nw) * Nq > 32) nw *= 2;
  return nw;
}

// One workgroup per GQA group, its G heads packed into the query columns of
// its waves: wave v holds heads v * pack .. v * pack + pack - 1 (those below
// G), column c of a wave row c % Nq of its head c / Nq.  Requires Nq <= 16
// (at least two heads per wave); one wave when G * Nq <= 32.
FA_HD inline fa_plan_t fa_make_packed_plan(int B, int Hq, int Hkv, int Nq, int Nk, int causal) {
  const int G = Hq / Hkv, nw = fa_packed_waves(G, Nq);
  fa_plan_t p = fa_make_plan(B, Hq, Hkv, Nq, Nk, causal, 32, nw);
  p.hw = p.G;
  p.pos = Nq;
  p.nqb = 1;
  p.nhg = 1;
  p.pack = (G + nw - 1) / nw;
  p.nwg = (long long)B * Hkv;
  p.xcd = fa_xcd_ways(p.nwg, 1, causal);
  return p;
}

// Split the keys of plan p into ranges of tps tiles of bc keys (nsplit =
// ceil(tiles / tps) ranges; tps >= 1).
FA_HD inline fa_plan_t fa_split_plan(fa_plan_t p, int tps, int bc) {
  const int tiles = (p.Nk + bc - 1) / bc;
  if (tps < 1) tps = 1;
  if (tps > tiles) tps = tiles;
  p.tps = tps;
  p.nsplit = (tiles + tps - 1) / tps;
  p.nwg = (long long)p.B * p.Hkv * p.nhg * p.nqb * p.nsplit;
  p.xcd = fa_xcd_ways(p.nwg, (long long)p.nqb * p.nsplit, p.causal);
  return p;
}

// Waves per workgroup: the largest power of two in [min_nw, max_nw] that
// still leaves at least `min_wg` workgroups; min_nw otherwise.
FA_HD inline fa_plan_t fa_choose_plan(int B, int Hq, int Hkv, int Nq, int Nk, int causal, int qpw,
                                      long long min_wg, int max_nw, int min_nw = 1) {
  for (int nw = max_nw; nw > min_nw; nw >>= 1) {
    fa_plan_t p = fa_make_plan(B, Hq, Hkv, Nq, Nk, causal, qpw, nw);
    if (p.nwg >= min_wg) return p;
  }
  return fa_make_plan(B, Hq, Hkv, Nq, Nk, causal, qpw, min_nw);
}

// Waves per workgroup of the bf16 and fp8 forward kernels.  A workgroup's
// K/V ring takes the same LDS whatever its wave count (bf16: 43 KB at
// d = 64, 75 KB at d = 128, 139 KB at d = 256; fp8: 21, 39, 75 KB), so LDS
// caps the workgroups per CU (3, 2, 1; 7, 4, 2) and too few waves per
// workgroup leave SIMDs idle: one-wave workgroups at d = 128 put 2 waves on
// a CU that holds 8.  Measured over 16 bf16 and 6 fp8 shapes (d = 64, 128,
// 256; 8 K to 524 K query rows), every choice below is the fastest or within
// 2.5 % of it, and up to 2.7x faster than the fewest waves that still leave
// 1024 workgroups:
//   bf16 d = 256: 4 waves, one workgroup per CU;
//   bf16 d = 128: 8 waves with at least 1024 workgroups, 2048 if causal
//     (each K/V tile then serves 256 query rows; causal work, which differs
//     between query blocks, needs the finer grid to balance: 4-wave
//     workgroups measured 6-11 % faster at 1024), else 4;
//   bf16 d = 64, fp8 d = 256: 4 waves with at least 512 workgroups, else 2;
//   fp8 d <= 128: 4 waves with at least 1024 workgroups, else 2, else 1
//     (4 to 7 one-wave workgroups share a CU, and smaller workgroups
//     balance causal work better).
FA_HD inline fa_plan_t fa_forward_plan(int B, int Hq, int Hkv, int Nq, int Nk, int causal, int d, int fp8,
                                       int qpw) {
  if (!fp8 && d == 256) return fa_make_plan(B, Hq, Hkv, Nq, Nk, causal, qpw, 4);
  if (!fp8 && d == 128) return fa_choose_plan(B, Hq, Hkv, Nq, Nk, causal, qpw, causal ? 2048 : 1024, 8, 4);
  if (fp8 && d <= 128) return fa_choose_plan(B, Hq, Hkv, Nq, Nk, causal, qpw, 1024, 4, 1);
  return fa_choose_plan(B, Hq, Hkv, Nq, Nk, causal, qpw, 512, 4, 2);
}

struct fa_work_t {
  int b, hkv, hq0, qpos0;  // batch, kv head, first query head, first query position
  int split;               // key range (0 without a split)
};

// Workgroup hardware id -> its work.  A bijection of [0, nwg) onto the
// (group, query block) pairs.
FA_HD inline fa_work_t fa_decode(const fa_plan_t& p, long long id) {
  unsigned L = (unsigned)fa_xcd_order(id, p.nwg, p.xcd);  // < 2^31 (fa_xcd_order)
  fa_work_t w;
  w.split = (int)(L % (unsigned)p.nsplit);
  L /= (unsigned)p.nsplit;
  unsigned g = L / (unsigned)p.nqb;
  int qi = (int)(L % (unsigned)p.nqb);
  if (p.causal) qi = p.nqb - 1 - qi;
  int hg = (int)(g % (unsigned)p.nhg);
  g /= (unsigned)p.nhg;
  w.hkv = (int)(g % (unsigned)p.Hkv);
  w.b = (int)(g / (unsigned)p.Hkv);
  w.hq0 = w.hkv * p.G + hg * p.hw;
  w.qpos0 = qi * p.pos;
  return w;
}

// Persistent grids: G workgroups (a multiple of 8, fewer than nwg) that
// each take several work items.  Workgroup g runs on XCD x = g % 8 and takes
// the ids the hardware would have handed to that XCD (x, x + 8, x + 16, ...,
// in that order), the U = G / 8 workgroups of the XCD sharing them in
// rounds of U: in round r workgroup u = g / 8 takes the u-th id of the round,
// or the (U-1-u)-th in odd rounds (a snake, so that over heaviest-first
// causal work each gets an even share).  Returns the id of round r, or ~0u
// past the last; a grid of nwg or more workgroups runs id = g (if g < nwg)
// in round 0.
FA_HD inline unsigned fa_persistent_item(unsigned G, long long nwg, unsigned g, unsigned r) {
  if ((long long)G >= nwg) return (r == 0 && (long long)g < nwg) ? g : ~0u;
  const unsigned x = g % 8, u = g / 8, U = G / 8;
  const unsigned id = x + 8 * (r * U + ((r & 1) ? U - 1 - u : u));  // < 2^31 + 8 G while r is in range
  return (long long)id < nwg ? id : ~0u;
}

// Number of key tiles of `bc` keys a workgroup starting at query position
// qpos0 must stream (causal: bottom-right aligned visibility j <= i + Nk - Nq).
FA_HD inline int fa_num_kv_tiles(const fa_plan_t& p, int qpos0, int bc) {
  int klast = p.Nk - 1;
  if (p.causal) {
    int qlast = qpos0 + p.pos - 1;
    if (qlast > p.Nq - 1) qlast = p.Nq - 1;
    int k = qlast + p.Nk - p.Nq;
    if (k < klast) klast = k;
  }
  return klast < 0 ? 0 : klast / bc + 1;
}

// Key tiles [t0, t1) of the workgroup's range, given its tile count nt
// (fa_num_kv_tiles); empty (t0 >= t1) when the range lies past every key
// the workgroup sees.
FA_HD inline void fa_split_tiles(const fa_plan_t& p, int split, int nt, int& t0, int& t1) {
  if (p.nsplit <= 1) {
    t0 = 0;
    t1 = nt;
    return;
  }
  t0 = split * p.tps;
  t1 = t0 + p.tps < nt ? t0 + p.tps : nt;
  if (t0 > t1) t0 = t1;
}

// ---------------------------------------------------------------- backward: key blocks
// The dK/dV kernel of the backward pass owns keys instead of queries: a
// wave keeps `kpw` consecutive keys of one key/value head (their K and V
// rows and their dK, dV accumulators) and streams the query rows of every
// query head of the GQA group past them, so that dK and dV, which sum over
// all those query heads, are each written by exactly one wave.  A workgroup
// holds `nw` waves over consecutive keys (`kpb` = kpw * nw keys), which
// share every query tile staged in LDS.  Workgroups are numbered
// group-major (group = batch, kv head) with the key blocks of a group
// consecutive, first key block first: with causal masking the first keys
// are seen by the most query rows, so the heaviest workgroups start first.
// The same XCD remap as above keeps the workgroups of one head on one L2
// (with causal masking, key blocks are runs that get heavier towards the
// start).
struct fa_kvplan_t {
  int B, Hq, Hkv, Nq, Nk;
  int causal;
  int G;     // Hq / Hkv
  int kpw;   // keys per wave
  int nw;    // waves per workgroup
  int kpb;   // keys per workgroup
  int nkb;   // key blocks per key/value head: ceil(Nk / kpb)
  int hsplit;  // parts the G query heads of a group are split into (divides G)
  int hps;     // query heads per part: G / hsplit
  int xcd;
  long long nwg;
};

FA_HD inline fa_kvplan_t fa_make_kvplan(int B, int Hq, int Hkv, int Nq, int Nk, int causal, int kpw, int nw) {
  fa_kvplan_t p;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Nq = Nq; p.Nk = Nk; p.causal = causal;
  p.G = Hq / Hkv;
  p.kpw = kpw;
  p.nw = nw;
  p.kpb = kpw * nw;
  p.nkb = (Nk + p.kpb - 1) / p.kpb;
  p.hsplit = 1;
  p.hps = p.G;
  p.nwg = (long long)B * Hkv * p.nkb;
  p.xcd = fa_xcd_ways(p.nwg, p.nkb, causal);
  return p;
}

// Split the G query heads of every group of plan p into `parts` parts of
// G / parts heads (parts divides G): parts times the workgroups, each adding
// its heads' share of dK and dV into a partial sum.
FA_HD inline fa_kvplan_t fa_split_kvplan_heads(fa_kvplan_t p, int parts) {
  p.hsplit = parts;
  p.hps = p.G / parts;
  p.nwg = (long long)p.B * p.Hkv * p.nkb * parts;
  p.xcd = fa_xcd_ways(p.nwg, p.nkb, p.causal);
  return p;
}

struct fa_kvwork_t {
  int b, hkv, k0;  // batch, kv head, first key of the workgroup
  int hs;          // part of the group's query heads (0 without a split)
};

// Workgroup hardware id -> its key block and head part; a bijection of
// [0, nwg) onto the (group, head part, key block) triples, key blocks
// innermost, so that the workgroups of one (group, head part), which read
// the same query tiles, run on one XCD.
FA_HD inline fa_kvwork_t fa_kv_decode(const fa_kvplan_t& p, long long id) {
  const unsigned L = (unsigned)fa_xcd_order(id, p.nwg, p.xcd);  // < 2^31 (fa_xcd_order)
  fa_kvwork_t w;
  const unsigned gs = L / (unsigned)p.nkb;
  w.k0 = (int)(L % (unsigned)p.nkb) * p.kpb;
  w.hs = (int)(gs % (unsigned)p.hsplit);
  const unsigned g = gs / (unsigned)p.hsplit;
  w.hkv = (int)(g % (unsigned)p.Hkv);
  w.b = (int)(g / (unsigned)p.Hkv);
  return w;
}

// Query tiles of `bq` rows a key block starting at key k0 must visit: tiles
// [first, ntq).  Causal: query i sees key j iff j <= i + Nk - Nq, so rows
// below k0 - (Nk - Nq) see none of the block's keys.
FA_HD inline void fa_kv_query_tiles(const fa_kvplan_t& p, int k0, int bq, int& first, int& ntq) {
  ntq = (p.Nq + bq - 1) / bq;
  first = 0;
  if (p.causal) {
    const long long r = (long long)k0 - ((long long)p.Nk - p.Nq);
    if (r > 0) first = r >= p.Nq ? ntq : (int)(r / bq);
  }
}

#endif  // FA_PLAN_H

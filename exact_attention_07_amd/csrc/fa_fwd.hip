// fa_fwd.hip -- fused exact-attention forward kernels for gfx950 (MI355X).
//
// One kernel computes O = softmax(scale * Q K^T) V and LSE for a block of
// query rows without writing scores to memory ("FlashAttention (SV)",
// sections "Tiling och blockbearbetning", "Online-beräkning av Softmax",
// "Sammanslagning av operationer").
//
// Mapping onto CDNA4
// ------------------
// * Each wave owns 32 query rows and keeps their Q fragments in VGPRs for
//   the whole pass; at d <= 128 a wave needs at most 256 VGPRs, so two waves
//   share each SIMD.
// * A workgroup of NW waves (plan.h; up to 8 at d = 128, one workgroup per
//   CU, so that every K/V tile fetched from L2 serves 256 query rows) streams
//   K/V tiles of BC = 64 keys through LDS.  Tiles are copied HBM -> LDS
//   directly with buffer_load_dwordx4 ... lds (16 B per lane, bounds-checked
//   by the buffer resource so rows past the end read as zero), double
//   buffered, so the copy of a tile overlaps the math on the tiles before it
//   (the asynchronous next-block load of "FlashAttention-3 — 闪电注意力-3",
//   section on minimising memory operations).  LDS rows are padded so that
//   the K row reads and the transposed V reads hit distinct banks with plain
//   "lane base + constant" addresses.
// * Scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16:
//   the accumulator then holds, in each lane, 16 keys of ONE query, so a row
//   maximum is an in-lane max plus one v_permlane32_swap, and the fp32
//   accumulator registers, rounded to bf16, are directly the B operand of
//   O^T += V^T P^T (no LDS round trip for P).  V^T fragments come from LDS
//   with ds_read_b64_tr_b16.
// * Each wave software-pipelines three streams per key tile: the MFMAs of
//   the next tile's scores, the exponentials of this tile, and the MFMAs of
//   the previous tile's P V, one MFMA per chunk with an equal share of the
//   softmax work, so the exponentials overlap the matrix products (the
//   softmax / matrix-product overlap FlashAttention-3 obtains with ping-pong
//   warpgroups, "FlashAttention-3 — 闪电注意力-3", section on asynchrony).
// * Online softmax in log2 units (c = scale * log2 e folded into one FMA).
//   The output is rescaled only when some row's running maximum has grown by
//   more than TAU = 8 over the reference maximum its exponentials use
//   ("FlashAttention-4震撼发布", first algorithmic improvement); stored
//   probabilities are then at most 2^8, and the result is exact for any TAU.
// * Row sums are kept per lane and combined once in the epilogue, and the
//   1/l normalisation is deferred to the epilogue (fewer non-matmul
//   operations, "FlashAttention-4震撼发布", FlashAttention-2 list).
// * Causal masking: key tiles entirely above the diagonal are never loaded,
//   tiles entirely below run unmasked, only tiles that cross it (or the
//   ragged end of the keys) apply the mask.
//
// fp32 inputs: every fp32 operand x is split into bf16 parts hi = bf16(x),
// lo = bf16(x - hi); products use hi*hi + hi*lo + lo*hi (about 2^-16
// relative), both for Q K^T and for P V.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "fa_device.h"
#include "fa_exp2.h"
#include "fa_frag.h"
#include "fa_kernels.h"
#include "plan.h"

namespace fa {

template <int D, bool F32>
struct Cfg {
  // query rows per wave: 32, so that (d <= 128) the whole wave state fits in
  // 256 VGPRs and two waves share a SIMD
  static constexpr int QPW = 32;
  static constexpr int WAVES_PER_SIMD = (D <= 128) ? 2 : 1;
  static constexpr int QB = QPW / 32;  // 32-row query blocks per wave
  static constexpr int KB = BC / 32;   // 32-key blocks per tile
  static constexpr int DS = D / 16;    // k-steps of S^T = K Q^T
  static constexpr int DB = D / 32;    // 32-row blocks of O^T
  static constexpr int PS = BC / 16;   // k-steps of O^T += V^T P^T
  // LDS tiles: BC rows of D bf16 (CPR 16-byte data slots), each row padded so
  // that the fragment reads hit distinct banks of the 64 x 4-byte banks with
  // plain "lane base + constant" addresses:
  //  * K rows: one padding slot.  A b128 read serves 16 lanes at a time,
  //    here one 16-byte chunk of 16 consecutive rows; a row stride of an odd
  //    multiple of 4 banks puts them on 16 distinct groups of 4 banks.
  //  * V rows: four padding slots.  A ds_read_b64_tr_b16 serves 32 lanes at
  //    a time, here 64 bytes (16 banks) of each of 4 consecutive rows; a row
  //    stride of 16 (or 48) banks modulo 64 makes the four rows disjoint.
  static constexpr int CPR = D / 8;                    // data slots per row
  static constexpr int SPR_K = CPR + 1;                // slots per K row
  static constexpr int SPR_V = CPR + 4;                // slots per V row
  static constexpr int RSK = SPR_K * 16, RSV = SPR_V * 16;  // LDS row strides, bytes
  static constexpr int TILE_K = BC * RSK, TILE_V = BC * RSV;  // bytes of one tile
  static_assert((RSK / 4) % 8 == 4, "K rows: odd multiple of 4 banks");
  static_assert((RSV / 4) % 64 == 16 || (RSV / 4) % 64 == 48, "V rows: 16 or 48 banks");
};

__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    __bf16 h = (__bf16)x[e];
    hi[e] = h;
    lo[e] = (__bf16)(x[e] - (float)h);
  }
}

// fp32 tile -> (hi, lo) bf16 tiles through registers (synchronous); rows past
// Nk are zero.
template <int D, int SPR>
__device__ __forceinline__ void copy_tile_f32(const float* src, int j0, int Nk, LDS_AS char* tile_hi,
                                              LDS_AS char* tile_lo) {
  constexpr int CPR = D / 8;
  for (int sl = threadIdx.x; sl < BC * SPR; sl += blockDim.x) {
    const int r = sl / SPR, pp = sl % SPR;
    if (pp >= CPR) continue;
    bf16x8 hi = {}, lo = {};
    if (j0 + r < Nk) {
      const f32x4* g = (const f32x4*)(src + (size_t)(j0 + r) * D + pp * 8);
      f32x4 a = g[0], b = g[1];
      float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      split8(x, hi, lo);
    }
    *(LDS_AS bf16x8*)(tile_hi + sl * 16) = hi;
    *(LDS_AS bf16x8*)(tile_lo + sl * 16) = lo;
  }
}

// fp32 operands: each is split into bf16 hi + lo parts as it is staged
// (synchronously, one tile at a time) and every product uses hi*hi + hi*lo +
// lo*hi on the same MFMA layouts as the bf16 path.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fa_fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                          const float* __restrict__ V, float* __restrict__ O,
                                                          float* __restrict__ LSE, fa_plan_t p, float c) {
  using C = Cfg<D, true>;
  constexpr int KB = C::KB, DS = C::DS, DB = C::DB, PS = C::PS, RSK = C::RSK, RSV = C::RSV;
  __shared__ __attribute__((aligned(1024))) char smem_[2 * C::TILE_K + 2 * C::TILE_V];
  LDS_AS char* const smem = (LDS_AS char*)smem_;
  LDS_AS char* const kt = smem;
  LDS_AS char* const ktl = smem + C::TILE_K;
  LDS_AS char* const vt = smem + 2 * C::TILE_K;
  LDS_AS char* const vtl = smem + 2 * C::TILE_K + C::TILE_V;

  const fa_work_t w = fa_decode(p, blockIdx.x);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hq = w.hq0 + wave % p.hw;
  const int q0w = w.qpos0 + (wave / p.hw) * 32;
  const int Nq = p.Nq, Nk = p.Nk;
  const int ntiles = fa_num_kv_tiles(p, w.qpos0, BC);

  const bool live = q0w < Nq;
  const int qlast_w = min(Nq - 1, q0w + 31);
  const int klast_w = CAUSAL ? min(Nk - 1, qlast_w + Nk - Nq) : Nk - 1;
  const int kfull_w = CAUSAL ? min(Nk - 1, q0w + Nk - Nq) : Nk - 1;

  const size_t qoff = (size_t)(w.b * p.Hq + hq) * Nq * D;
  const size_t kvoff = (size_t)(w.b * p.Hkv + w.hkv) * Nk * D;

  bf16x8 qf[DS], qlo[DS];
  {
    const int qrow = min(q0w + (lane & 31), Nq - 1);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const f32x4* g = (const f32x4*)(Q + qoff + (size_t)qrow * D + ds * 16 + (lane >> 5) * 8);
      f32x4 a = g[0], b = g[1];
      float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      split8(x, qf[ds], qlo[ds]);
    }
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x16){};
  float m_ref = NEG_INF, m_run = NEG_INF, lsum = 0.f;
  const int koff_l = k_lane_off<RSK>(lane);
  const int voff_l = v_lane_off<RSV>(lane);

  for (int j = 0; j < ntiles; ++j) {
    const int j0 = j * BC;
    __syncthreads();
    copy_tile_f32<D, C::SPR_K>(K + kvoff, j0, Nk, kt, ktl);
    copy_tile_f32<D, C::SPR_V>(V + kvoff, j0, Nk, vt, vtl);
    __syncthreads();
    if (!live || j0 > klast_w) continue;  // wave-uniform: nothing visible to this wave

    // ---- S^T = K Q^T (three partial products)
    f32x16 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s[kb] = (f32x16){};
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int off = koff_l + kb * 32 * RSK + ds * 32;
        const bf16x8 kh = lds_b128(kt + off), kl = lds_b128(ktl + off);
        s[kb] = mfma(kh, qf[ds], s[kb]);
        s[kb] = mfma(kh, qlo[ds], s[kb]);
        s[kb] = mfma(kl, qf[ds], s[kb]);
      }

    if (j0 + BC - 1 > kfull_w) {
      const int query = q0w + (lane & 31);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int kmax = (CAUSAL ? min(Nk - 1, query + Nk - Nq) : Nk - 1) - j0 - kb * 32 - (lane >> 5) * 4;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if ((i >> 2) * 8 + (i & 3) > kmax) s[kb][i] = NEG_INF;
      }
    }

    float mx = NEG_INF;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    m_run = fmaxf(m_run, xhalf_max(mx) * c);
    if (__ballot(m_run > m_ref + TAU)) {
      const float alpha = (m_run == NEG_INF) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_run);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      m_ref = m_run;
    }

    // ---- P = 2^(S c - m_ref) split into bf16 hi + lo; row sums from the fp32 P
    const float mu = (m_ref == NEG_INF) ? 0.f : m_ref;
    bf16x8 ph[PS], pl[PS];
    float part = 0.f;
#pragma unroll
    for (int ps = 0; ps < PS; ++ps) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[ps >> 1][(ps & 1) * 8 + e], c, -mu));
        part += x[e];
      }
      split8(x, ph[ps], pl[ps]);
    }
    lsum += part;

    // ---- O^T += V^T P^T (three partial products)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int ps = 0; ps < PS; ++ps) {
        const bf16x8 vh = v_frag<RSV>(vt + voff_l, ps, db), vl = v_frag<RSV>(vtl + voff_l, ps, db);
        o[db] = mfma(vh, ph[ps], o[db]);
        o[db] = mfma(vh, pl[ps], o[db]);
        o[db] = mfma(vl, ph[ps], o[db]);
      }
  }

  if (!live) return;
  const float lt = xhalf_sum(lsum);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  const int query = q0w + (lane & 31);
  if (query >= Nq) return;
  const size_t orow = qoff + (size_t)query * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      f32x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = o[db][i4 * 4 + e] * inv;
      *(f32x4*)(O + orow + db * 32 + i4 * 8 + (lane >> 5) * 4) = r;
    }
  if (LSE != nullptr && lane < 32)
    LSE[(size_t)(w.b * p.Hq + hq) * Nq + query] = lt > 0.f ? (m_ref + log2f(lt)) * LN2 : NEG_INF;
}

// ---------------------------------------------------------------- bf16 kernel helpers

// Scores of one wave for one key tile (S^T blocks [kb][qb]).
template <int D>
struct Scores {
  using C = Cfg<D, false>;
  f32x16 v[C::KB][C::QB];
};

// S^T = K Q^T for one tile, fully in one go (prologue).
template <int D>
__device__ __forceinline__ void scores_full(Scores<D>& s, LDS_AS const char* klane,
                                            const bf16x8 (&qf)[Cfg<D, false>::QB][Cfg<D, false>::DS]) {
  using C = Cfg<D, false>;
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) s.v[kb][qb] = (f32x16){};
#pragma unroll
  for (int ds = 0; ds < C::DS; ++ds)
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
      const bf16x8 kf = lds_b128(klane + kb * 32 * C::RSK + ds * 32);
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) s.v[kb][qb] = mfma(kf, qf[qb][ds], s.v[kb][qb]);
    }
}

// Mask keys past the visible range of each query (tiles that cross the
// causal diagonal or the end of the keys only).
// query: the row of the lane's query column.
template <int D, bool CAUSAL>
__device__ __forceinline__ void mask_scores(Scores<D>& s, int j0, int query, int Nq, int Nk, int kend, int lane) {
  using C = Cfg<D, false>;
  static_assert(C::QB == 1, "one 32-row query block per wave");
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      const int klim = min(kend, CAUSAL ? min(Nk, query + Nk - Nq + 1) : Nk);  // keys < klim are visible
      const int kmax = klim - 1 - j0 - kb * 32 - (lane >> 5) * 4;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if ((i >> 2) * 8 + (i & 3) > kmax) s.v[kb][qb][i] = NEG_INF;
    }
}

// ---------------------------------------------------------------- bf16 kernel
// Iteration j of a wave interleaves three independent streams, one MFMA per
// chunk: the MFMAs of S_{j+1} = K_{j+1} Q^T, the exponentials of tile j, and
// the MFMAs of O^T += V_{j-1}^T P_{j-1}^T.  Every MFMA thus carries the same
// share of softmax work (one score per MFMA at d = 128), rather than all of
// it next to the S MFMAs and none next to the P V MFMAs.
// The lazy rescale of tile j runs after P_{j-1} V_{j-1} has entered O, so O
// and P_j always refer to the same reference maximum.
//
// LDS ring (two slots each): iteration j reads K_{j+1} and V_{j-1} and
// refills the slots of K_j and V_{j-2} with K_{j+2} and V_j; every copy has
// one iteration to land before the barrier that publishes it.
//
// One work item (fa_decode of id) per call; a persistent workgroup calls it
// once per item, with a barrier in between (the LDS ring is reused).
// EMU: how many of every four exponentials run as the FMA-pipe polynomial
// exp2_poly (fa_exp2.h) instead of v_exp_f32 (0 for fa_fwd).
template <int D, bool CAUSAL, int NW, int EMU>
__device__ __forceinline__ void fwd_bf16_item(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                              const __bf16* __restrict__ V, __bf16* __restrict__ O,
                                              float* __restrict__ LSE, const fa_plan_t& p, float c,
                                              float* __restrict__ OWS, float* __restrict__ LWS, unsigned id) {
  using C = Cfg<D, false>;
  constexpr int KB = C::KB, DS = C::DS, DB = C::DB, PS = C::PS, RSK = C::RSK, RSV = C::RSV;
  static_assert(C::QB == 1, "one 32-row query block per wave");
  constexpr int NMF = DS * KB;        // MFMAs of one S^T tile
  constexpr int NPV = DB * PS;        // MFMAs of one P V product
  static_assert(NMF == NPV, "S and P V streams alternate");
  // At d <= 128 the MFMAs go in pairs of the same product, S S P V P V
  // (0.4-0.65 % faster than strict alternation at d = 128, on two boxes);
  // at d = 256 they alternate P V, S (1.3 % faster there).
  constexpr int GRP = D == 256 ? 1 : 2;
  static_assert(NMF % GRP == 0, "whole groups of each product");
  constexpr int NSC = KB * 16;        // scores per lane per tile
  constexpr int NCH = NMF + NPV;      // chunks of the fused phase
  constexpr int KPF = 2, VPF = 2;     // LDS fragment reads in flight per stream
  using CopyK = CopyPlan<D, NW, C::SPR_K>;
  using CopyV = CopyPlan<D, NW, C::SPR_V>;
  // Ring slot t & 1 of tile t.  Every slot is an array of its own: a copy
  // into one slot then provably cannot alias the reads of the other, and the
  // compiler does not wait for the copies in flight before each transposed
  // V read (it does for reads of the same array).
  __shared__ __attribute__((aligned(1024))) char lk0_[C::TILE_K];
  __shared__ __attribute__((aligned(1024))) char lk1_[C::TILE_K];
  __shared__ __attribute__((aligned(1024))) char lv0_[C::TILE_V];
  __shared__ __attribute__((aligned(1024))) char lv1_[C::TILE_V];
  __shared__ __attribute__((aligned(1024))) char lsp_[1024];
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  auto kslot = [&](auto par) { return (LDS_AS char*)(decltype(par)::value == 0 ? lk0_ : lk1_); };
  auto vslot = [&](auto par) { return (LDS_AS char*)(decltype(par)::value == 0 ? lv0_ : lv1_); };
  LDS_AS char* const spare = (LDS_AS char*)lsp_;

  const fa_work_t w = fa_decode(p, id);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hq = w.hq0 + wave % p.hw;
  const int q0w = w.qpos0 + (wave / p.hw) * 32;
  const int Nq = p.Nq, Nk = p.Nk;
  const int nt = fa_num_kv_tiles(p, w.qpos0, BC);
  // key tiles [t0, t1) of this workgroup's range (all of them without a split)
  int t0, t1;
  fa_split_tiles(p, w.split, nt, t0, t1);
  const int kend = t1 * BC;  // keys past the range are masked like invisible ones

  const bool live = q0w < Nq;
  const int qlast_w = min(Nq - 1, q0w + 31);
  const int klast_w = CAUSAL ? min(Nk - 1, qlast_w + Nk - Nq) : Nk - 1;
  const int kfull_w = min(kend - 1, CAUSAL ? min(Nk - 1, q0w + Nk - Nq) : Nk - 1);
  // tiles of the range this wave computes (t0 .. t0 + ntw - 1)
  const int ntw = (live && klast_w >= 0) ? max(0, min(t1, klast_w / BC + 1) - t0) : 0;

  const size_t kvoff = (size_t)(w.b * p.Hkv + w.hkv) * Nk * D;
  // the lane's query column: head hq_l, row q_l (valid_l: a real query).
  // Packed plans hold, in column c of wave v, row c % Nq of head
  // hq0 + v * pack + c / Nq; every wave then covers rows 0 .. Nq - 1 of its
  // heads, so the wave-level limits above hold unchanged.
  const int col = lane & 31;
  int hq_l = hq, q_l = q0w + col;
  bool valid_l = q_l < Nq;
  if (p.pack > 1) {
    const int hh = col / Nq, head = wave * p.pack + hh;
    valid_l = hh < p.pack && head < p.G;
    hq_l = w.hq0 + (valid_l ? head : 0);
    q_l = valid_l ? col - hh * Nq : 0;
  }
  const size_t qrow0 = (size_t)(w.b * p.Hq + hq_l) * Nq;  // first row of the lane's head

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x16){};
  // lsum: row sum of the fp32 probabilities (the LSE).  At d = 256 also
  // lsumq, the row sum of the bf16-rounded probabilities that multiply V,
  // which normalises O: O is then a convex combination of V rows with
  // exactly the weights applied, without the error (rounding of P) x |V| that
  // dominates rows with one or two heavy keys.  It costs one dot2 per pair of
  // probabilities: measured +1 % at d = 256, +4.6 % at d = 128, where O is
  // normalised by lsum (see the error bound where the tolerance is stated).
  constexpr bool QSUM = D == 256;
  float m_ref = NEG_INF, m_run = NEG_INF, lsum = 0.f, lsumq = 0.f;

  // A range without key tiles (causal rows that see no key, or a key range
  // past every visible key of the workgroup's rows; uniform over the
  // workgroup) loads and copies nothing: the epilogue writes O = 0 and
  // LSE = -inf straight away.
  if (t1 > t0) {
  bf16x8 qf[1][DS];
  {
    const int qrow = min(q_l, Nq - 1);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qf[0][ds] = *(const bf16x8*)(Q + (qrow0 + qrow) * D + ds * 16 + (lane >> 5) * 8);
  }

  const int koff_l = k_lane_off<RSK>(lane);
  const int voff_l = v_lane_off<RSV>(lane);
  CopyK cpk;
  CopyV cpv;
  cpk.init(wave, lane);
  cpv.init(wave, lane);
  const __amdgpu_buffer_rsrc_t kres = CopyK::rsrc(K + kvoff, Nk), vres = CopyV::rsrc(V + kvoff, Nk);
  const int kv_bytes = Nk * (D * 2);
  auto tile_off = [&](int t) { return t < t1 ? t * (BC * D * 2) : kv_bytes; };
  // Copy instruction i of this wave in iteration j (of parity par): K_{j+2}
  // into K slot par, then V_j into V slot par.  The instructions are spread
  // over the chunks of the iteration rather than issued in one burst.
  constexpr int NCP = CopyK::MI + CopyV::MI;
  auto copy_one = [&](int j, auto par, int i) {
    if (i < CopyK::MI) cpk.issue_one(kres, tile_off(j + 2), kslot(par), spare, wave, i);
    else cpv.issue_one(vres, tile_off(j), vslot(par), spare, wave, i - CopyK::MI);
  };
  auto copy_all = [&](int j, auto par) {
    cpk.issue_all(kres, tile_off(j + 2), kslot(par), spare, wave);
    cpv.issue_all(vres, tile_off(j), vslot(par), spare, wave);
  };

  // prologue: K_{t0}, K_{t0+1}, zeros into V slot 1, which iteration 0 reads
  // (its P V product then adds 0 x 0); S_{t0}
  cpk.issue_all(kres, tile_off(t0), kslot(P0{}), spare, wave);
  cpk.issue_all(kres, tile_off(t0 + 1), kslot(P1{}), spare, wave);
  cpv.issue_all(vres, kv_bytes, vslot(P1{}), spare, wave);
  vm_wait<0>();
  __syncthreads();
  Scores<D> sa, sb;
  if (ntw > 0) scores_full<D>(sa, kslot(P0{}) + koff_l, qf);

  // probabilities of one tile, bf16 pairs packed per dword (B operand of P V)
  struct Probs {
    u32x4 v[PS];
  };
  Probs pa, pb;
#pragma unroll
  for (int ps = 0; ps < PS; ++ps) pb.v[ps] = (u32x4){0u, 0u, 0u, 0u};

  const bf16x2 ones2 = {(__bf16)1.0f, (__bf16)1.0f};
  // the pair (sc - 1, sc) of odd sc: its odd member into the row sum, the
  // pair packed into its P dword (and, with QSUM, into the rounded row sum)
  auto flush_pair = [&](Probs& pf, int sc, float& part1, float even, float odd, float& partq) {
    const int skb = sc / 16, si = sc % 16;
    part1 += odd;
    const unsigned pk = pack_bf16(even, odd);
    pf.v[skb * 2 + si / 8][(si % 8) / 2] = pk;
    if constexpr (QSUM) partq = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), ones2, partq, false);
  };
  // score sc = (kb, i) of s: exponential against mu, row-sum part, packed
  // into the P dword of its pair.  At d = 128, one score per MFMA, the
  // row-sum adds and the packing run one score late, so that no instruction
  // waits on the exponential just issued (1.4 % faster there; at d = 64 and
  // 256, with two MFMAs per score, 0.4-0.5 % slower): the even member of a
  // pair goes into the row sum at the odd member, the pair at the next even
  // score (flush_pair; after the last score the caller flushes it).
  // Otherwise the odd member of a pair adds itself and packs the pair.
  constexpr bool DEFER = D == 128;
  auto arg_of = [&](const Scores<D>& s, int sc, float mu) {
    return __builtin_fmaf(s.v[sc / 16][0][sc % 16], c, -mu);
  };
  auto score = [&](const Scores<D>& s, Probs& pf, int sc, float mu, float& part0, float& part1, float& even,
                   float& odd, float& partq, float& next_arg) {
    const int skb = sc / 16, si = sc % 16;
    float arg;
    if constexpr (DEFER) {
      // the argument was formed one score ahead
      arg = next_arg;
      if (sc + 1 < NSC) next_arg = arg_of(s, sc + 1, mu);
    } else {
      arg = arg_of(s, sc, mu);
    }
    const float pv = (EMU > 0 && (sc & 3) >= 4 - EMU) ? exp2_poly(arg) : __builtin_amdgcn_exp2f(arg);
    if constexpr (DEFER) {
      if (sc & 1) {
        part0 += even;
        odd = pv;
      } else {
        if (sc > 0) flush_pair(pf, sc - 1, part1, even, odd, partq);
        even = pv;
      }
    } else if (sc & 1) {
      flush_pair(pf, sc, part1, even, pv, partq);
    } else {
      part0 += pv;
      even = pv;
    }
  };

  // the exponentials of tile j (scores in s, probabilities into pf), the
  // MFMAs of S_{j+1} (into sn) and of O += V_{j-1} P_{j-1} (pprev).  At
  // j = t0 + ntw (the wave's last P V product) tile j lies past every key
  // the wave's queries see in this range, so the mask turns all its scores
  // into -inf and its exponentials contribute nothing.
  // (par = j & 1: K_{j+1} and V_{j-1} are read from the slots 1 - par.)
  auto fused = [&](int j, auto par, Scores<D>& s, Scores<D>& sn, Probs& pf, const Probs& pprev) {
    using other = std::integral_constant<int, 1 - decltype(par)::value>;
    const int j0 = j * BC;
    LDS_AS const char* knext = kslot(other{}) + koff_l;
    LDS_AS const char* vprev = vslot(other{}) + voff_l;
    bf16x8 kbuf[KPF], vbuf[VPF];
#pragma unroll
    for (int t = 0; t < KPF; ++t) kbuf[t] = lds_b128(knext + (t % KB) * 32 * RSK + (t / KB) * 32);
#pragma unroll
    for (int t = 0; t < VPF; ++t) vbuf[t] = v_frag<RSV>(vprev, t / DB, t % DB);
    if (j0 + BC - 1 > kfull_w) mask_scores<D, CAUSAL>(s, j0, q_l, Nq, Nk, kend, lane);

    float mu = (m_ref == NEG_INF) ? 0.f : m_ref;
    float part0 = 0.f, part1 = 0.f, even = 0.f, odd = 0.f, partq = 0.f;
    float next_arg = DEFER ? arg_of(s, 0, mu) : 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sn.v[kb][0] = (f32x16){};
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      const int m = (ch / (2 * GRP)) * GRP + (ch % GRP);
      if (GRP > 1 ? (ch % (2 * GRP)) < GRP : (ch % 2) == 1) {
        // S_{j+1}: MFMA m, reading the K fragment KPF MFMAs ahead
        const int ds = m / KB, kb = m % KB;
        sn.v[kb][0] = mfma(kbuf[m % KPF], qf[0][ds], sn.v[kb][0]);
        if (m + KPF < NMF) kbuf[m % KPF] = lds_b128(knext + ((m + KPF) % KB) * 32 * RSK + ((m + KPF) / KB) * 32);
      } else {
        // O += V_{j-1} P_{j-1}: MFMA m (k-step m / DB, d-block m % DB)
        const int ps = m / DB, db = m % DB;
        o[db] = mfma(vbuf[m % VPF], __builtin_bit_cast(bf16x8, pprev.v[ps]), o[db]);
        if (m + VPF < NPV) vbuf[m % VPF] = v_frag<RSV>(vprev, (m + VPF) / DB, (m + VPF) % DB);
      }
      // scores [ch * NSC / NCH, (ch + 1) * NSC / NCH)
#pragma unroll
      for (int sc = ch * NSC / NCH; sc < (ch + 1) * NSC / NCH; ++sc)
        score(s, pf, sc, mu, part0, part1, even, odd, partq, next_arg);
      // the NCP copy instructions over the first half of the chunks, so each
      // has more than half an iteration to land (against spreading them over
      // all chunks: +1 % at d = 128, +5 % at d = 64 causal, +10 % at d = 256;
      // all in the first chunk or the first quarter measured slower at d = 256)
#pragma unroll
      for (int i = ch * NCP / (NCH / 2); i < (ch + 1) * NCP / (NCH / 2) && i < NCP; ++i) copy_one(j, par, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (DEFER) flush_pair(pf, NSC - 1, part1, even, odd, partq);
    float part = part0 + part1;

    // slow path: if some probability may exceed 2^TAU (a lane's partial row
    // sum does), or a row has no reference yet, form the row maximum; when
    // it grew by more than TAU, rescale O (which already holds
    // P_{j-1} V_{j-1}) and l and redo the exponentials.  Otherwise every
    // probability is at most 2^TAU and the reference maximum stands, exactly
    // as the max-first rule would decide, and the exponentials already taken
    // are the ones it gives.
    if (__ballot(!(part <= TAU_EXP2) || m_ref == NEG_INF)) {
      float mx = NEG_INF;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s.v[kb][0][i]);
      m_run = fmaxf(m_run, xhalf_max(mx) * c);
      if (__ballot(m_run > m_ref + TAU)) {
        const float alpha = (m_run == NEG_INF) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_run);
        lsum *= alpha;
        lsumq *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
        m_ref = m_run;
        mu = (m_ref == NEG_INF) ? 0.f : m_ref;
        part0 = part1 = partq = 0.f;
        next_arg = arg_of(s, 0, mu);
#pragma unroll
        for (int sc = 0; sc < NSC; ++sc) score(s, pf, sc, mu, part0, part1, even, odd, partq, next_arg);
        if constexpr (DEFER) flush_pair(pf, NSC - 1, part1, even, odd, partq);
        part = part0 + part1;
      }
    }
    lsum += part;
    lsumq += partq;
  };

  // one code path for every iteration a wave takes part in (j <= ntw);
  // waves past their last tile only keep the barriers and copies going
  // iteration i of the range handles tile j = t0 + i
  auto iteration = [&](int i, auto par, Scores<D>& s, Scores<D>& sn, Probs& pf, Probs& pprev) {
    const int j = t0 + i;
    vm_wait<0>();
    __syncthreads();
    if (i <= ntw && ntw > 0) {
      fused(j, par, s, sn, pf, pprev);
    } else {
      copy_all(j, par);
    }
  };
  // iterations 0 .. n-1 (n = t1 - t0); score and probability buffers
  // alternate (unrolled by two)
  const int n = t1 - t0;
  for (int i = 0; i <= n - 1; i += 2) {
    iteration(i, P0{}, sa, sb, pa, pb);
    if (i + 1 <= n - 1) iteration(i + 1, P1{}, sb, sa, pb, pa);
  }
  // iteration n only adds O += V_{t1-1} P_{t1-1} (no tile follows: no
  // scores, exponentials or copies); its buffers by the parity of n
  vm_wait<0>();
  __syncthreads();
  if (n <= ntw) {
    LDS_AS const char* vprev = ((n & 1) ? (LDS_AS const char*)lv0_ : (LDS_AS const char*)lv1_) + voff_l;
    Probs pp;
#pragma unroll
    for (int ps = 0; ps < PS; ++ps) pp.v[ps] = (n & 1) ? pa.v[ps] : pb.v[ps];
    bf16x8 vbuf[VPF];
#pragma unroll
    for (int t = 0; t < VPF; ++t) vbuf[t] = v_frag<RSV>(vprev, t / DB, t % DB);
#pragma unroll
    for (int m = 0; m < NPV; ++m) {
      const int ps = m / DB, db = m % DB;
      o[db] = mfma(vbuf[m % VPF], __builtin_bit_cast(bf16x8, pp.v[ps]), o[db]);
      if (m + VPF < NPV) vbuf[m % VPF] = v_frag<RSV>(vprev, (m + VPF) / DB, (m + VPF) % DB);
    }
  }
  }  // t1 > t0

  // ---- epilogue: O / l, LSE = ln2 * (m_ref + log2 l); with a key split, the
  // range's partial result (fp32) goes to the workspace for the merge
  if (!live) return;
  const float lt = xhalf_sum(lsum);
  const float ltq = QSUM ? xhalf_sum(lsumq) : lt;
  const float inv = ltq > 0.f ? 1.0f / ltq : 0.f;
  if (!valid_l) return;
  const float lse_row = lt > 0.f ? (m_ref + log2f(lt)) * LN2 : NEG_INF;
  if (p.nsplit > 1) {
    const size_t row = (size_t)w.split * p.B * p.Hq * Nq + qrow0 + q_l;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = o[db][i4 * 4 + e] * inv;
        *(f32x4*)(OWS + row * D + db * 32 + i4 * 8 + (lane >> 5) * 4) = r;
      }
    if (lane < 32) LWS[row] = lse_row;
    return;
  }
  const size_t orow = (qrow0 + q_l) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = db * 32 + i4 * 8 + (lane >> 5) * 4;
      bf16x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = (__bf16)(o[db][i4 * 4 + e] * inv);
      *(bf16x4*)(O + orow + d0) = r;
    }
  if (LSE != nullptr && lane < 32) LSE[qrow0 + q_l] = lse_row;
}

// A grid of p.nwg workgroups runs one work item each.  The kernels that hold
// a whole CU per workgroup (8 waves at d = 128, 4 at d = 256) also run as a
// persistent grid of one workgroup per CU (fa_persistent_item), and so do the
// causal 4-wave kernels at d = 64 and 128, two workgroups per CU: each
// workgroup then takes its items one after another, so a CU's next item
// starts without a new workgroup's dispatch, and the snake order over the
// heaviest-first causal work gives every workgroup an even share.
template <int D, bool CAUSAL, int NW, int EMU>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(Cfg<D, false>::WAVES_PER_SIMD)))
void fa_fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                        __bf16* __restrict__ O, float* __restrict__ LSE, fa_plan_t p, float c,
                        float* __restrict__ OWS, float* __restrict__ LWS) {
  if constexpr (!((D == 128 && NW == 8) || (D == 256 && NW == 4) || (CAUSAL && NW == 4 && (D == 64 || D == 128)))) {
    fwd_bf16_item<D, CAUSAL, NW, EMU>(Q, K, V, O, LSE, p, c, OWS, LWS, blockIdx.x);
  } else {
    for (unsigned r = 0;; ++r) {
      const unsigned id = fa_persistent_item(gridDim.x, p.nwg, blockIdx.x, r);
      if (id == ~0u) break;
      if (r > 0) __syncthreads();  // every wave is done with the last item's LDS
      fwd_bf16_item<D, CAUSAL, NW, EMU>(Q, K, V, O, LSE, p, c, OWS, LWS, id);
    }
  }
}

// ---------------------------------------------------------------- launchers
// Every variant is instantiated explicitly (implicit instantiation through
// the launch expression alone does not always emit the host-side stub).
#define FA_INST_F32(DD, CC)                                                                               \
  template __global__ void fa_fwd_f32_kernel<DD, CC>(const float* __restrict__, const float* __restrict__,       \
                                                     const float* __restrict__, float* __restrict__,             \
                                                     float* __restrict__, fa_plan_t, float);
#define FA_F32_VARIANTS(X) X(64, false) X(64, true) X(128, false) X(128, true) X(256, false) X(256, true)
FA_F32_VARIANTS(FA_INST_F32)
#define FA_INST_BF16_E(DD, CC, NN, EE)                                                                    \
  template __global__ void fa_fwd_bf16_kernel<DD, CC, NN, EE>(const __bf16* __restrict__, const __bf16* __restrict__, \
                                                              const __bf16* __restrict__, __bf16* __restrict__,     \
                                                              float* __restrict__, fa_plan_t, float,                \
                                                              float* __restrict__, float* __restrict__);
#define FA_INST_BF16(DD, CC, NN) FA_INST_BF16_E(DD, CC, NN, 0)
// (head dim, causal, waves per workgroup)
#define FA_BF16_VARIANTS(X)                                                                                \
  X(64, false, 1) X(64, false, 2) X(64, false, 4) X(64, true, 1) X(64, true, 2) X(64, true, 4)              \
  X(128, false, 1) X(128, false, 2) X(128, false, 4) X(128, false, 8)                                       \
  X(128, true, 1) X(128, true, 2) X(128, true, 4) X(128, true, 8)                                           \
  X(256, false, 1) X(256, false, 2) X(256, false, 4) X(256, true, 1) X(256, true, 2) X(256, true, 4)
FA_BF16_VARIANTS(FA_INST_BF16)
// the same at d = 64 and 128 with a quarter (EMU 1) or half (EMU 2) of the
// exponentials on the FMA pipe (fa_fwd_exp2_emulated)
#define FA_BF16_EMU_VARIANTS(X, EE)                                                                        \
  X(64, false, 1, EE) X(64, false, 2, EE) X(64, false, 4, EE) X(64, true, 1, EE) X(64, true, 2, EE)        \
  X(64, true, 4, EE) X(128, false, 1, EE) X(128, false, 2, EE) X(128, false, 4, EE) X(128, false, 8, EE)   \
  X(128, true, 1, EE) X(128, true, 2, EE) X(128, true, 4, EE) X(128, true, 8, EE)
FA_BF16_EMU_VARIANTS(FA_INST_BF16_E, 1)
FA_BF16_EMU_VARIANTS(FA_INST_BF16_E, 2)

// ---------------------------------------------------------------- merge of key ranges
// One wave per output row (b, h, i): with L = ln sum_s exp(lse_s),
// O = sum_s exp(lse_s - L) O_s and LSE = L ("FlashAttention (SV)", section
// "Online-beräkning av Softmax": block statistics combine exactly).  Ranges
// that saw no key (lse_s = -inf) weigh nothing; rows with none get O = 0 and
// LSE = -inf.  Lane t handles columns t*D/64 .. +D/64.
template <int D>
__global__ __launch_bounds__(64) void fa_merge_kernel(const float* __restrict__ OWS, const float* __restrict__ LWS,
                                                      __bf16* __restrict__ O, float* __restrict__ LSE, int nsplit,
                                                      long long rows) {
  constexpr int EPL = D / 64;
  const long long row = blockIdx.x;
  const int lane = threadIdx.x;
  float m = NEG_INF;
  for (int sp = 0; sp < nsplit; ++sp) m = fmaxf(m, LWS[sp * rows + row]);
  float acc[EPL] = {};
  float tot = 0.f;
  if (m != NEG_INF) {
    for (int sp = 0; sp < nsplit; ++sp) {
      const float l = LWS[sp * rows + row];
      const float wgt = __builtin_amdgcn_exp2f((l - m) * 1.4426950408889634f);  // exp(-inf) = 0
      tot += wgt;
      const float* src = OWS + ((size_t)sp * rows + row) * D + lane * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = __builtin_fmaf(wgt, src[e], acc[e]);
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) O[row * D + lane * EPL + e] = (__bf16)(acc[e] * inv);
  if (LSE != nullptr && lane == 0) LSE[row] = tot > 0.f ? m + logf(tot) : NEG_INF;
}

hipError_t launch_merge(const float* ows, const float* lws, void* o, float* lse, int nsplit, long long rows, int d,
                        hipStream_t stream) {
  if (rows < 1 || rows > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)rows);
  if (d == 64) hipLaunchKernelGGL(fa_merge_kernel<64>, grid, dim3(64), 0, stream, ows, lws, (__bf16*)o, lse, nsplit, rows);
  else if (d == 128) hipLaunchKernelGGL(fa_merge_kernel<128>, grid, dim3(64), 0, stream, ows, lws, (__bf16*)o, lse, nsplit, rows);
  else if (d == 256) hipLaunchKernelGGL(fa_merge_kernel<256>, grid, dim3(64), 0, stream, ows, lws, (__bf16*)o, lse, nsplit, rows);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

int queries_per_wave(int, int) { return 32; }

// The CU count of each device, read once: 0 = not read yet, -1 = unknown.
// Launching threads may race to fill an entry; each stores the same value,
// and the atomic makes the race benign (no torn or stale-forever reads).
static std::atomic<int> g_cus[64];

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int cus = g_cus[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    cus = n >= 8 ? n / 8 * 8 : -1;
    g_cus[dev].store(cus, std::memory_order_relaxed);
  }
  return cus > 0 ? cus : 0;
}

unsigned persistent_grid(long long nwg, int per_cu) {
  const int cus = cu_count();
  const long long g = (long long)cus * per_cu;
  return (cus > 0 && nwg > g) ? (unsigned)g : (unsigned)nwg;
}

// Workgroups of a bf16 forward launch: p.nwg, or a persistent grid for the
// kernels that hold a whole CU per workgroup and for the causal 4-wave ones
// that fit two per CU (LDS and registers; non-causal items are all alike,
// and measured 1.8 % slower at d = 64).
static unsigned fwd_grid(const fa_plan_t& p, int d) {
  if ((d == 128 && p.nw == 8) || (d == 256 && p.nw == 4)) return persistent_grid(p.nwg);
  if ((d == 128 || d == 64) && p.nw == 4 && p.causal) return persistent_grid(p.nwg, 2);
  return (unsigned)p.nwg;
}

hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, const fa_plan_t& p, int d,
                      float c, int f32, float* ows, float* lws, hipStream_t stream, int emu) {
#define FA_CASE_F32(DD, CC)                                                                               \
  if (f32 && d == DD && (p.causal != 0) == CC) {                                                        \
    hipLaunchKernelGGL((fa_fwd_f32_kernel<DD, CC>), dim3((unsigned)p.nwg), dim3(256), 0, stream, (const float*)q, \
                       (const float*)k, (const float*)v, (float*)o, lse, p, c);                        \
    return hipGetLastError();                                                                           \
  }
#define FA_CASE_BF16_E(DD, CC, NN, EE)                                                                 \
  if (!f32 && emu == EE && d == DD && (p.causal != 0) == CC && p.nw == NN) {                            \
    hipLaunchKernelGGL((fa_fwd_bf16_kernel<DD, CC, NN, EE>), dim3(fwd_grid(p, d)), dim3(64 * NN), 0, stream,  \
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, p, c, ows, lws); \
    return hipGetLastError();                                                                           \
  }
#define FA_CASE_BF16(DD, CC, NN) FA_CASE_BF16_E(DD, CC, NN, 0)
  if (f32 && p.nsplit > 1) return hipErrorInvalidValue;  // the fp32 kernel has no key split
  FA_F32_VARIANTS(FA_CASE_F32)
  FA_BF16_VARIANTS(FA_CASE_BF16)
  FA_BF16_EMU_VARIANTS(FA_CASE_BF16_E, 1)
  FA_BF16_EMU_VARIANTS(FA_CASE_BF16_E, 2)
#undef FA_CASE_F32
#undef FA_CASE_BF16
#undef FA_CASE_BF16_E
  return hipErrorInvalidValue;
}

}  // namespace fa

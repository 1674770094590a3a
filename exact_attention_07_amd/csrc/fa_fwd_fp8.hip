// fa_fwd_fp8.hip -- fused exact-attention forward kernel on e4m3 operands
// for gfx950 (MI355X).
//
// The FP8 form of the fused forward pass ("FlashAttention-3 — 闪电注意力-3",
// sections on Hopper's FP8 support and on low precision): both matrix
// products run on 8-bit floating point, whose dense peak is twice that of
// bf16, with fp32 accumulation.  The operands come from fa_fp8_prepare (Q
// and K rotated by a signed Hadamard matrix and quantised with one scale per
// tensor, V quantised and stored transposed).  The structure is that of the
// bf16 kernel (the Q codes carry the softmax scale in log2 units, so the
// scores need no multiply): 32 query rows per wave with their Q codes resident in VGPRs,
// K and V^T tiles of 64 keys copied HBM -> LDS with bounds-checked buffer
// loads, double buffered; scores transposed (S^T = K Q^T) so that a lane
// holds the scores of one query; the online softmax with the output
// rescaled only when a row maximum grows by more than TAU; causal tiles
// above the diagonal skipped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"
#include "plan.h"

namespace fa {

// ---------------------------------------------------------------- fp8 kernel
// e4m3 operands (from fa_fp8_prepare) on v_mfma_f32_32x32x64_f8f6f4: each
// lane supplies 32 bytes of the 64-long contraction; the product pairs byte j
// of lane l of A with byte j of lane l' of B when l/32 == l'/32, so both
// operands only need the same (half, byte) <-> k assignment.
//   S^T = K8 Q8^T: half h of a lane holds d = ks*64 + h*32 .. +31.
//   O^T += V8^T P8^T: byte j of half h of the P fragment is the probability
//   of S^T accumulator block j/16, register j%16, i.e. key
//   (j/16)*32 + (j%16/4)*8 + h*4 + j%4; fa_fp8_prepare stores V^T with the
//   keys of each 64-key block in exactly this order, so a lane's 32 bytes of
//   a V^T row are contiguous.
// Scores come out of the matrix core in the units the exponentials take:
// fa_fp8_prepare quantises Q with the softmax scale and log2 e folded in and
// with power-of-two scales s_q, s_k, so x = s_q s_k (K8 Q8^T) is exactly the
// score in log2 units; the MFMA applies 2^(e_q + e_k) through its E8M0 scale
// operands, and the first k-step of each block starts its accumulator at
// -mu (mu the row's reference maximum), so the exponential takes the MFMA
// result as it is: no multiply-add per score.  The epilogue multiplies O by
// s_v / l.  P (at most 2^TAU = 256 < 448) is quantised unscaled.
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// the same with E8M0 scales (biased exponents: 127 = 2^0) on A and B
__device__ __forceinline__ f32x16 mfma_fp8_scaled(i32x8 a, i32x8 b, f32x16 c, int ea, int eb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
}
__device__ __forceinline__ i32x8 lds_b256(LDS_AS const char* p) {
  const i32x4 a = *(LDS_AS const i32x4*)p, b = *(LDS_AS const i32x4*)(p + 16);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Copy plan of a tile of ROWS rows; an LDS row holds CPR 16-byte data slots
// and SPR - CPR padding slots; rows are row_stride bytes apart in memory.
template <int ROWS, int CPR, int SPR, int NW>
struct TileCopy {
  static constexpr int SLOTS = ROWS * SPR;
  static_assert(SLOTS % 64 == 0, "a tile is a whole number of copy instructions");
  static constexpr int INS = SLOTS / 64;
  static constexpr int MI = (INS + NW - 1) / NW;
  static constexpr unsigned OUT_OF_RANGE = 0x7ffffff0u;
  unsigned goff[MI];
  __device__ __forceinline__ void init(int wave, int lane, int row_stride) {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int ins = i * NW + wave;
      const int sl = ins * 64 + lane;
      const int r = sl / SPR, pp = sl % SPR;
      goff[i] = (ins < INS && pp < CPR) ? (unsigned)(r * row_stride + pp * 16) : OUT_OF_RANGE;
    }
  }
  // copy instruction i of this wave for the tile at byte offset soff
  // (instructions past the tile, when NW does not divide INS, write into the
  // 1 KB block `spare`)
  __device__ __forceinline__ void issue_one(const __amdgpu_buffer_rsrc_t& rs, int soff, LDS_AS char* tile,
                                            LDS_AS char* spare, int wave, int i) const {
    const int ins = i * NW + wave;
    LDS_AS char* dst = (INS % NW == 0 || ins < INS) ? tile + ins * 1024 : spare;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)dst, 16, goff[i], soff, 0, 0);
  }
  __device__ __forceinline__ void issue_all(const __amdgpu_buffer_rsrc_t& rs, int soff, LDS_AS char* tile,
                                            LDS_AS char* spare, int wave) const {
#pragma unroll
    for (int i = 0; i < MI; ++i) issue_one(rs, soff, tile, spare, wave, i);
  }
};

// Iteration j of a wave interleaves three independent streams, one MFMA per
// chunk: the MFMAs of S_{j+1} = K_{j+1} Q^T, the exponentials (and e4m3
// packing) of tile j, and the MFMAs of O^T += V_{j-1}^T P_{j-1}^T.  Every
// chunk thus carries both matrix and vector work, so the matrix pipe of a
// SIMD is fed while its two waves take exponentials, instead of both waves
// taking all their exponentials, then all their products, in step.  The lazy
// rescale of tile j runs after P_{j-1} V_{j-1} has entered O, so O and P_j
// always refer to the same reference maximum.
// LDS ring (two slots each): iteration j reads K_{j+1} and V_{j-1} and
// refills the slots of K_j and V_{j-2} with K_{j+2} and V_j; each copy has
// one iteration to land before the barrier that publishes it.
template <int D, bool CAUSAL, int NW>
__device__ __forceinline__ void fwd_fp8_item(const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ K8,
                                             const uint8_t* __restrict__ V8T, const float* __restrict__ descale,
                                             __bf16* __restrict__ O, float* __restrict__ LSE, const fa_plan_t& p,
                                             unsigned item) {
  constexpr int KB = BC / 32;      // 32-key blocks per tile
  constexpr int KS = D / 64;       // k-steps of S^T
  constexpr int DB = D / 32;       // 32-row blocks of O^T
  constexpr int NMF = KB * KS;     // S^T MFMAs per tile
  constexpr int NPV = DB;          // P V MFMAs per tile (one per block covers the 64 keys)
  static_assert(NMF == NPV && NMF % 2 == 0, "S and P V streams alternate in pairs");
  constexpr int NCH = NMF + NPV;   // chunks of the fused phase
  constexpr int NSC = KB * 16;     // scores per lane per tile
  constexpr int SPC = NSC / NCH;   // scores per chunk
  static_assert(NSC % NCH == 0 && SPC % 2 == 0, "whole pairs of scores per chunk");
  constexpr int KPF = 2, VPF = 2;  // LDS fragment reads in flight per stream
  constexpr int RSK = D + 16;      // K8 LDS row stride (conflict-free for 16 consecutive keys)
  constexpr int RSV = 80;          // V8^T LDS row stride: 64 keys + 16 bytes
  constexpr int KTILE = BC * RSK, VTILE = D * RSV;
  using KCopy = TileCopy<BC, D / 16, D / 16 + 1, NW>;
  using VCopy = TileCopy<D, 4, 5, NW>;
  constexpr int NCP = KCopy::MI + VCopy::MI;
  // every ring slot is an array of its own, so that a copy into one slot
  // provably does not alias the reads of the other (the compiler then does
  // not wait for copies in flight before those reads)
  __shared__ __attribute__((aligned(1024))) char lk0_[KTILE];
  __shared__ __attribute__((aligned(1024))) char lk1_[KTILE];
  __shared__ __attribute__((aligned(1024))) char lv0_[VTILE];
  __shared__ __attribute__((aligned(1024))) char lv1_[VTILE];
  __shared__ __attribute__((aligned(1024))) char lsp_[1024];
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  auto kslot = [&](auto par) { return (LDS_AS char*)(decltype(par)::value == 0 ? lk0_ : lk1_); };
  auto vslot = [&](auto par) { return (LDS_AS char*)(decltype(par)::value == 0 ? lv0_ : lv1_); };
  LDS_AS char* const spare = (LDS_AS char*)lsp_;

  const fa_work_t w = fa_decode(p, item);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hq = w.hq0 + wave % p.hw;
  const int q0w = w.qpos0 + (wave / p.hw) * 32;
  const int Nq = p.Nq, Nk = p.Nk;
  const int Nkp = (Nk + BC - 1) / BC * BC;
  const int nt = fa_num_kv_tiles(p, w.qpos0, BC);
  const bool live = q0w < Nq;
  const int qlast_w = min(Nq - 1, q0w + 31);
  const int klast_w = CAUSAL ? min(Nk - 1, qlast_w + Nk - Nq) : Nk - 1;
  const int kfull_w = CAUSAL ? min(Nk - 1, q0w + Nk - Nq) : Nk - 1;
  // tiles this wave computes (0 .. ntw - 1)
  const int ntw = (live && klast_w >= 0) ? min(nt, klast_w / BC + 1) : 0;
  // E8M0 scales of the score product: the biased exponents of the power-of-two
  // s_q (for B, the Q codes) and s_k (for A, the K codes)
  const int e_q = __builtin_amdgcn_readfirstlane((int)((__float_as_uint(descale[0]) >> 23) & 0xff));
  const int e_k = __builtin_amdgcn_readfirstlane((int)((__float_as_uint(descale[1]) >> 23) & 0xff));
  const float sv = descale[2];

  const size_t qoff = (size_t)(w.b * p.Hq + hq) * Nq * D;
  const size_t koff = (size_t)(w.b * p.Hkv + w.hkv) * Nk * D;
  const size_t voff = (size_t)(w.b * p.Hkv + w.hkv) * D * Nkp;

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x16){};
  float m_ref = NEG_INF, m_run = NEG_INF, lsum = 0.f;

  // A workgroup without key tiles (causal rows that see no key) loads and
  // copies nothing: the epilogue writes O = 0 and LSE = -inf straight away.
  if (nt > 0) {
  // resident Q fragments: query lane%32, bytes ks*64 + (lane/32)*32 .. +31
  i32x8 qf[KS];
  {
    const int qrow = min(q0w + (lane & 31), Nq - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint8_t* g = Q8 + qoff + (size_t)qrow * D + ks * 64 + (lane >> 5) * 32;
      const i32x4 a = *(const i32x4*)g, b = *(const i32x4*)(g + 16);
      qf[ks] = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }

  const int koff_l = (lane & 31) * RSK + (lane >> 5) * 32;
  const int voff_l = (lane & 31) * RSV + (lane >> 5) * 32;
  KCopy kc;
  VCopy vc;
  kc.init(wave, lane, D);
  vc.init(wave, lane, Nkp);
  const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc((void*)(K8 + koff), (short)0, Nk * D, 0x00020000);
  const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc((void*)(V8T + voff), (short)0, D * Nkp, 0x00020000);
  // byte offsets of tile t (past the last tile: past the buffer, reads zeros)
  auto tile_k = [&](int t) { return t < nt ? t * BC * D : Nk * D; };
  auto tile_v = [&](int t) { return t < nt ? t * BC : D * Nkp; };
  // Without a causal mask the key tiles are taken in a rotated order: pass
  // i < nt takes tile (i + rot) mod nt, with rot spread evenly over the
  // head's query blocks, so that the workgroups of one head, which run side
  // by side, each fetch a different tile at a time instead of all waiting
  // on the same first fetch (measured 1-1.5 % faster on the non-causal
  // d = 128 workload, though L2 then fetches some tiles again).  Passes
  // from nt on are past the last tile.
  const int rot = CAUSAL ? 0 : (int)((unsigned long long)(w.qpos0 / p.pos) * (unsigned)nt / (unsigned)p.nqb);
  auto tile_of = [&](int i) { return (CAUSAL || i >= nt) ? i : (i + rot < nt ? i + rot : i + rot - nt); };
  // copy instruction i of this wave in iteration j (of parity par): K_{j+2}
  // into K slot par, then V_j into V slot par
  auto copy_one = [&](int j, auto par, int i) {
    if (i < KCopy::MI) kc.issue_one(kres, tile_k(tile_of(j + 2)), kslot(par), spare, wave, i);
    else vc.issue_one(vres, tile_v(tile_of(j)), vslot(par), spare, wave, i - KCopy::MI);
  };
  auto copy_all = [&](int j, auto par) {
    kc.issue_all(kres, tile_k(tile_of(j + 2)), kslot(par), spare, wave);
    vc.issue_all(vres, tile_v(tile_of(j)), vslot(par), spare, wave);
  };

  // prologue: K_0, K_1, zeros into V slot 1, which iteration 0 reads (its
  // P V product then adds 0 x 0); S_0
  kc.issue_all(kres, tile_k(tile_of(0)), kslot(P0{}), spare, wave);
  kc.issue_all(kres, tile_k(tile_of(1)), kslot(P1{}), spare, wave);
  vc.issue_all(vres, D * Nkp, vslot(P1{}), spare, wave);
  vm_wait<0>();
  __syncthreads();
  f32x16 sa[KB], sb[KB];
  if (ntw > 0) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sa[kb] = (f32x16){};
#pragma unroll
    for (int t = 0; t < NMF; ++t)
      sa[t % KB] = mfma_fp8_scaled(lds_b256(kslot(P0{}) + koff_l + (t % KB) * 32 * RSK + (t / KB) * 64), qf[t / KB],
                                   sa[t % KB], e_k, e_q);
  }
  // the accumulator start of a score block: -mu of the lane's row (mu = the
  // reference maximum, 0 while the row has none)
  f32x16 negmu;
#pragma unroll
  for (int i = 0; i < 16; ++i) negmu[i] = 0.f;
  i32x8 pa, pb;
#pragma unroll
  for (int i = 0; i < 8; ++i) pb[i] = 0;

  // score sc of s (already x - mu): exponential and row-sum part.  Packing
  // into byte sc of the P fragment (the odd member of a pair packs the pair
  // into its half-dword) takes one of three forms:
  //   HOLD: the probability is kept in pvs and the whole tile is packed
  //     after the slow-path check (pack_held);
  //   PACK: packed where it is formed;
  //   PIN:  as PACK, with the low half written over the dword's stale
  //     contents (which the high half then replaces) instead of over a zero,
  //     and an empty asm taking each finished dword as an input where it is
  //     formed, so that the compiler keeps the packing beside the MFMAs.
  // Measured: packing beside the MFMAs is 2-3.5 % faster on causal shapes
  // and at d = 256, holding 1-1.5 % faster on the non-causal d = 128
  // workload, hence the choice below.
  enum { HOLD, PACK, PIN };
  float pvs[NSC];
  auto score = [&](const f32x16 (&s)[KB], i32x8& pf, int sc, float& part0, float& part1, float& even, int mode) {
    const float pv = __builtin_amdgcn_exp2f(s[sc / 16][sc % 16]);
    if (sc & 1) {
      part1 = sc == 1 ? pv : part1 + pv;
      const int pp = sc / 2;
      if (mode == HOLD) {
        pvs[sc] = pv;
      } else if (pp & 1) {
        pf[pp / 2] = __builtin_amdgcn_cvt_pk_fp8_f32(even, pv, pf[pp / 2], true);
        if (mode == PIN) asm volatile("" ::"v"(pf[pp / 2]));
      } else {
        pf[pp / 2] = __builtin_amdgcn_cvt_pk_fp8_f32(even, pv, mode == PIN ? pf[pp / 2] : 0, false);
      }
    } else {
      part0 = sc == 0 ? pv : part0 + pv;
      even = pv;
      if (mode == HOLD) pvs[sc] = pv;
    }
  };
  // (each dword's two halves are both written, so its old contents do not matter)
  auto pack_held = [&](i32x8& pf) {
#pragma unroll
    for (int pp = 0; pp < NSC / 2; ++pp)
      pf[pp / 2] = (pp & 1) ? __builtin_amdgcn_cvt_pk_fp8_f32(pvs[2 * pp], pvs[2 * pp + 1], pf[pp / 2], true)
                            : __builtin_amdgcn_cvt_pk_fp8_f32(pvs[2 * pp], pvs[2 * pp + 1], pf[pp / 2], false);
  };
  constexpr bool HELD = !CAUSAL && D == 128;
  constexpr int FIRST = HELD ? HOLD : PIN, AGAIN = HELD ? HOLD : PACK;

  // the exponentials of tile j (scores in s, probabilities into pf), the
  // MFMAs of S_{j+1} (into sn) and of O += V_{j-1} P_{j-1} (pprev).  At the
  // wave's tile ntw, past its last key, the mask turns every score into -inf.
  auto fused = [&](int j, auto par, f32x16 (&s)[KB], f32x16 (&sn)[KB], i32x8& pf, const i32x8& pprev) {
    using other = std::integral_constant<int, 1 - decltype(par)::value>;
    const int j0 = tile_of(j) * BC;
    LDS_AS const char* knext = kslot(other{}) + koff_l;
    LDS_AS const char* vprev = vslot(other{}) + voff_l;
    i32x8 kbuf[KPF], vbuf[VPF];
#pragma unroll
    for (int t = 0; t < KPF; ++t) kbuf[t] = lds_b256(knext + (t % KB) * 32 * RSK + (t / KB) * 64);
#pragma unroll
    for (int t = 0; t < VPF; ++t) vbuf[t] = lds_b256(vprev + t * 32 * RSV);
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
    // s holds x - mu: it was started at -mu, or shifted to it when the
    // slow path moved the reference
    const float mu = (m_ref == NEG_INF) ? 0.f : m_ref;
    float part0 = 0.f, part1 = 0.f, even = 0.f;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      // the MFMAs in pairs of the same product, S S P V P V (0.75 % faster
      // than strict alternation on the non-causal d = 128 workload)
      const int m = (ch / 4) * 2 + (ch % 2);
      if ((ch % 4) < 2) {
        // S_{j+1}: MFMA m (k-step m / KB, key block m % KB)
        sn[m % KB] = mfma_fp8_scaled(kbuf[m % KPF], qf[m / KB], (m / KB == 0) ? negmu : sn[m % KB], e_k, e_q);
        if (m + KPF < NMF)
          kbuf[m % KPF] = lds_b256(knext + ((m + KPF) % KB) * 32 * RSK + ((m + KPF) / KB) * 64);
      } else {
        // O += V_{j-1} P_{j-1}: MFMA m (d-block m)
        o[m] = mfma_fp8(vbuf[m % VPF], pprev, o[m]);
        if (m + VPF < NPV) vbuf[m % VPF] = lds_b256(vprev + (m + VPF) * 32 * RSV);
      }
#pragma unroll
      for (int sc = ch * SPC; sc < (ch + 1) * SPC; ++sc) score(s, pf, sc, part0, part1, even, FIRST);
      // the copy instructions over the first half of the chunks: each then
      // has more than half an iteration to land (measured 1-2 % faster than
      // spreading them over all chunks)
#pragma unroll
      for (int i = 0; i < NCP; ++i)
        if (ch == i * (NCH / 2) / NCP) copy_one(j, par, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    float part = part0 + part1;
    // slow path, as in the bf16 kernel: if some probability may exceed
    // 2^TAU (a lane's partial row sum does) or a row has no reference yet,
    // form the row maximum; when it grew by more than TAU, rescale O (which
    // already holds P_{j-1} V_{j-1}) and l, shift both score buffers (this
    // tile's and S_{j+1}, complete by now) to the new reference, start later
    // blocks at it and redo the exponentials.  When the reference stands the
    // exponentials already taken are the ones it gives.
    if (__ballot(!(part <= TAU_EXP2) || m_ref == NEG_INF)) {
      float mx = NEG_INF;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      m_run = fmaxf(m_run, xhalf_max(mx) + mu);
      if (__ballot(m_run > m_ref + TAU)) {
        const float alpha = (m_run == NEG_INF) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_run);
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
        m_ref = m_run;
        const float mu2 = (m_ref == NEG_INF) ? 0.f : m_ref;
        const float dm = mu - mu2;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          s[kb] += dm;
          sn[kb] += dm;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) negmu[i] = -mu2;
#pragma unroll
        for (int sc = 0; sc < NSC; ++sc) score(s, pf, sc, part0, part1, even, AGAIN);
        part = part0 + part1;
      }
    }
    if constexpr (HELD) pack_held(pf);
    lsum += part;
  };

  // one code path for every iteration a wave takes part in (j <= ntw);
  // waves past their last tile only keep the barriers and copies going
  auto iteration = [&](int j, auto par, f32x16 (&s)[KB], f32x16 (&sn)[KB], i32x8& pf, i32x8& pprev) {
    vm_wait<0>();
    __syncthreads();
    if (j <= ntw && ntw > 0) fused(j, par, s, sn, pf, pprev);
    else copy_all(j, par);
  };
  for (int j = 0; j <= nt - 1; j += 2) {
    iteration(j, P0{}, sa, sb, pa, pb);
    if (j + 1 <= nt - 1) iteration(j + 1, P1{}, sb, sa, pb, pa);
  }
  // iteration nt only adds O += V_{nt-1} P_{nt-1}; it also waits for the
  // last copies (zeros past the final tile), which must land before the
  // workgroup's LDS can pass to another workgroup
  vm_wait<0>();
  __syncthreads();
  if (nt <= ntw) {
    LDS_AS const char* vprev = ((nt & 1) ? (LDS_AS const char*)lv0_ : (LDS_AS const char*)lv1_) + voff_l;
    const i32x8 pp = (nt & 1) ? pa : pb;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = mfma_fp8(lds_b256(vprev + db * 32 * RSV), pp, o[db]);
  }
  }  // nt > 0

  if (!live) return;
  const float lt = xhalf_sum(lsum);
  const float inv = lt > 0.f ? sv / lt : 0.f;
  const int query = q0w + (lane & 31);
  if (query >= Nq) return;
  const size_t orow = qoff + (size_t)query * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      bf16x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = (__bf16)(o[db][i4 * 4 + e] * inv);
      *(bf16x4*)(O + orow + db * 32 + i4 * 8 + (lane >> 5) * 4) = r;
    }
  if (LSE != nullptr && lane < 32)
    LSE[(size_t)(w.b * p.Hq + hq) * Nq + query] = lt > 0.f ? (m_ref + log2f(lt)) * LN2 : NEG_INF;
}

// The causal 4-wave kernels (two workgroups per CU at d <= 128, one at
// d = 256) and the non-causal 4-wave d = 256 kernel, which holds a CU alone,
// run as persistent grids (fa_persistent_item): each workgroup takes work
// items in rounds, in the snake order that evens out causal work, so a CU's
// next item starts without a new workgroup's dispatch.  The other forms run
// one item per workgroup.
template <int D, bool CAUSAL, int NW>
constexpr bool fp8_persistent() {
  return NW == 4 && (CAUSAL || D == 256);
}

template <int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1)))
void fa_fwd_fp8_kernel(const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ K8,
                       const uint8_t* __restrict__ V8T, const float* __restrict__ descale,
                       __bf16* __restrict__ O, float* __restrict__ LSE, fa_plan_t p) {
  if constexpr (!fp8_persistent<D, CAUSAL, NW>()) {
    fwd_fp8_item<D, CAUSAL, NW>(Q8, K8, V8T, descale, O, LSE, p, blockIdx.x);
  } else {
    for (unsigned r = 0;; ++r) {
      const unsigned id = fa_persistent_item(gridDim.x, p.nwg, blockIdx.x, r);
      if (id == ~0u) break;
      if (r > 0) __syncthreads();  // every wave is done with the last item's LDS
      fwd_fp8_item<D, CAUSAL, NW>(Q8, K8, V8T, descale, O, LSE, p, id);
    }
  }
}

// ---------------------------------------------------------------- launcher
#define FA_INST_FP8(DD, CC, NN)                                                                              \
  template __global__ void fa_fwd_fp8_kernel<DD, CC, NN>(const uint8_t* __restrict__, const uint8_t* __restrict__, \
                                                         const uint8_t* __restrict__, const float* __restrict__,   \
                                                         __bf16* __restrict__, float* __restrict__, fa_plan_t);
#define FA_FP8_VARIANTS(X)                                                                                  \
  X(64, false, 1) X(64, false, 2) X(64, false, 4) X(64, true, 1) X(64, true, 2) X(64, true, 4)              \
  X(128, false, 1) X(128, false, 2) X(128, false, 4) X(128, true, 1) X(128, true, 2) X(128, true, 4)        \
  X(256, false, 1) X(256, false, 2) X(256, false, 4) X(256, true, 1) X(256, true, 2) X(256, true, 4)
FA_FP8_VARIANTS(FA_INST_FP8)

// workgroups of a launch: the persistent forms above get one or two per CU
static unsigned fp8_grid(const fa_plan_t& p, int d) {
  if (p.nw == 4 && (p.causal || d == 256)) return persistent_grid(p.nwg, d == 256 ? 1 : 2);
  return (unsigned)p.nwg;
}

hipError_t launch_fwd_fp8(const void* q8, const void* k8, const void* v8t, const float* descale, void* o, float* lse,
                          const fa_plan_t& p, int d, hipStream_t stream) {
#define FA_CASE_FP8(DD, CC, NN)                                                                           \
  if (d == DD && (p.causal != 0) == CC && p.nw == NN) {                                                 \
    hipLaunchKernelGGL((fa_fwd_fp8_kernel<DD, CC, NN>), dim3(fp8_grid(p, d)), dim3(64 * NN), 0, stream,      \
                       (const uint8_t*)q8, (const uint8_t*)k8, (const uint8_t*)v8t, descale, (__bf16*)o, lse, p); \
    return hipGetLastError();                                                                           \
  }
  FA_FP8_VARIANTS(FA_CASE_FP8)
#undef FA_CASE_FP8
  return hipErrorInvalidValue;
}

}  // namespace fa

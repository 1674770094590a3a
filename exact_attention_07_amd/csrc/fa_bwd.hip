// fa_bwd.hip -- backward pass of exact attention for gfx950 (MI355X):
// gradients dQ, dK, dV for an upstream gradient dO, recomputing the
// probabilities from Q, K and the saved log-sum-exp instead of storing them.
//
// The pages report training speed-ups ("FlashAttention-4震撼发布",
// FlashAttention-2 list; "FlashAttention (SV)", section "Empiriska
// resultat") but print no backward algorithm.  What is computed is the
// derivative of the definition ("FlashAttention (SV)", section
// "Problematik med standard-attention"), with P = softmax(scale Q K^T):
//
//     dV = P^T dO          dP = dO V^T          D_i = sum_c dO_ic O_ic
//     dS = P o (dP - D)    dQ = scale dS K      dK  = scale dS^T Q
//
// and P_ij = 2^(scale log2(e) q_i.k_j - LSE_i log2(e)) is rebuilt tile by
// tile from the forward pass's LSE, the same tiling that keeps the N x N
// matrices out of memory in the forward pass ("FlashAttention (SV)",
// sections "Tiling och blockbearbetning" and "Sammanslagning av
// operationer").  D_i = sum_j P_ij dP_ij equals the row dot product of dO and
// O, so it needs no pass over the keys.
//
// Two kernels, no atomics:
// * fa_bwd_dq_kernel: the forward kernel's shape.  A wave owns 32 query rows
//   of one head (Q and dO fragments in VGPRs), streams the K/V tiles of its
//   key/value head through LDS and accumulates dQ^T += K^T dS^T.  Its
//   prologue also forms D_i and LSE_i log2(e) of its rows and stores them
//   (8 bytes per row) for the second kernel.
// * fa_bwd_dkdv_kernel: the transposed shape.  A wave owns 64 keys of one
//   key/value head (K and V fragments in VGPRs, dK^T and dV^T accumulators)
//   and streams the query tiles of every query head of its GQA group through
//   LDS: S = Q K^T, dP = dO V^T, then dV^T += dO^T P and dK^T += Q^T dS.  The
//   sum over the group's query heads stays inside the wave, so dK and dV are
//   written once, without atomics.
// Per 64 x 64 block of (queries, keys) the two kernels run 7 matrix products
// where 5 would do (S and dP are formed in both); in exchange nothing is
// accumulated across workgroups, which on an 8-XCD chip (one L2 per XCD)
// would need device-scope atomics on dQ from every key block.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_frag.h"
#include "fa_kernels.h"
#include "plan.h"

namespace fa {

constexpr float LOG2E_F = 1.44269504088896341f;

template <int D>
struct BwdCfg {
  static constexpr int DS = D / 16;  // k-steps over the head dimension
  static constexpr int DB = D / 32;  // 32-row blocks of a D-row accumulator
  static constexpr int KB = BC / 32; // 32-row blocks of a 64-row tile
  static constexpr int PS = BC / 16; // k-steps over a 64-row tile
  static constexpr int CPR = D / 8;  // 16-byte data slots per row
  // LDS row strides: an odd number of 16-byte slots per row (one padding
  // slot).  Tiles read both as row fragments and transposed (K in the dQ
  // kernel, Q and dO in the dK/dV kernel) also store their rows in perm16
  // order (fa_frag.h), which makes both kinds of read free of bank conflicts.
  static constexpr int SPR_X = CPR + 1;
  static constexpr int SPR_R = CPR + 1;
  static constexpr int RSX = SPR_X * 16, RSR = SPR_R * 16;
  static constexpr int TILE_X = BC * RSX, TILE_R = BC * RSR;
  static_assert((RSX / 4) % 8 == 4 && (RSR / 4) % 8 == 4, "row fragments: odd multiple of 4 banks");
};

using P0 = std::integral_constant<int, 0>;
using P1 = std::integral_constant<int, 1>;

// ---------------------------------------------------------------- dQ (and D, LSE log2 e)
// Wave state: Q and dO rows as B operands (lane: query row lane % 32, 8
// consecutive columns per k-step), dQ^T accumulators (d x 32).  Per key tile:
//   S^T  = K Q^T   (A = K rows from LDS)       dP^T = V dO^T (A = V rows)
//   P^T  = 2^(S^T c - L2), dS^T = P^T o (dP^T - D), packed to bf16 in place
//   dQ^T += K^T dS^T (A = K^T, transposed LDS reads in the row order of the
//   S^T accumulator)
// One work item (fa_decode of id) per call; a persistent workgroup calls it
// once per item, with a barrier in between (the LDS ring is reused).
template <int D, bool CAUSAL, int NW>
__device__ __forceinline__ void bwd_dq_item(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                            const __bf16* __restrict__ V, const __bf16* __restrict__ O,
                                            const __bf16* __restrict__ dO, const float* __restrict__ LSE,
                                            float* __restrict__ LD, __bf16* __restrict__ dQ, const fa_plan_t& p,
                                            float c, float scale, unsigned id) {
  using C = BwdCfg<D>;
  constexpr int DS = C::DS, DB = C::DB, KB = C::KB, PS = C::PS, RSX = C::RSX, RSR = C::RSR;
  using CopyK = CopyPlan<D, NW, C::SPR_X, true>;
  using CopyV = CopyPlan<D, NW, C::SPR_R>;
  __shared__ __attribute__((aligned(1024))) char lk0_[C::TILE_X];
  __shared__ __attribute__((aligned(1024))) char lk1_[C::TILE_X];
  __shared__ __attribute__((aligned(1024))) char lv0_[C::TILE_R];
  __shared__ __attribute__((aligned(1024))) char lv1_[C::TILE_R];
  __shared__ __attribute__((aligned(1024))) char lsp_[1024];
  auto kslot = [&](auto par) { return (LDS_AS char*)(decltype(par)::value == 0 ? lk0_ : lk1_); };
  auto vslot = [&](auto par) { return (LDS_AS char*)(decltype(par)::value == 0 ? lv0_ : lv1_); };
  LDS_AS char* const spare = (LDS_AS char*)lsp_;

  const fa_work_t w = fa_decode(p, id);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hq = w.hq0 + wave % p.hw;
  const int q0w = w.qpos0 + (wave / p.hw) * 32;
  const int Nq = p.Nq, Nk = p.Nk, off = Nk - Nq;
  const int nt = fa_num_kv_tiles(p, w.qpos0, BC);
  const bool live = q0w < Nq;
  const int qlast_w = min(Nq - 1, q0w + 31);
  const int klast_w = CAUSAL ? min(Nk - 1, qlast_w + off) : Nk - 1;
  const int kfull_w = CAUSAL ? min(Nk - 1, q0w + off) : Nk - 1;
  const int ntw = (live && klast_w >= 0) ? klast_w / BC + 1 : 0;  // tiles this wave computes

  const size_t rowbase = (size_t)(w.b * p.Hq + hq) * Nq;
  const size_t qoff = rowbase * D;
  const size_t kvoff = (size_t)(w.b * p.Hkv + w.hkv) * Nk * D;
  const int query = q0w + (lane & 31);
  const int qrow = min(query, Nq - 1);

  // Q, dO fragments; D = rowsum(dO o O) from the same loads of O
  bf16x8 qf[DS], dof[DS];
  float L2, Drow;
  {
    float dsum = 0.f;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const size_t e0 = qoff + (size_t)qrow * D + ds * 16 + (lane >> 5) * 8;
      qf[ds] = *(const bf16x8*)(Q + e0);
      dof[ds] = *(const bf16x8*)(dO + e0);
      const bf16x8 of = *(const bf16x8*)(O + e0);
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum = __builtin_fmaf((float)dof[ds][e], (float)of[e], dsum);
    }
    Drow = xhalf_sum(dsum);
    const float lse = LSE[rowbase + qrow];
    // a row that sees no key (LSE = -inf) has every score masked; 0 keeps
    // 2^(-inf - L2) = 0 free of NaN
    L2 = lse == NEG_INF ? 0.f : lse * LOG2E_F;
    if (live && lane < 32 && query < Nq) {
      LD[(rowbase + query) * 2] = L2;
      LD[(rowbase + query) * 2 + 1] = Drow;
    }
  }

  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = (f32x16){};

  const int koff_l = k_lane_off_p<RSX>(lane), voff_l = k_lane_off<RSR>(lane), toff_l = v_lane_off_p<RSX>(lane);
  CopyK cpk;
  CopyV cpv;
  cpk.init(wave, lane);
  cpv.init(wave, lane);
  const __amdgpu_buffer_rsrc_t kres = CopyK::rsrc(K + kvoff, Nk), vres = CopyV::rsrc(V + kvoff, Nk);
  auto issue = [&](int j, auto par) {
    cpk.issue_all(kres, j * (BC * D * 2), kslot(par), spare, wave);
    cpv.issue_all(vres, j * (BC * D * 2), vslot(par), spare, wave);
  };

  auto compute = [&](int j, auto par) {
    LDS_AS const char* kt = kslot(par);
    LDS_AS const char* vt = vslot(par);
    const int j0 = j * BC;
    f32x16 st[KB], dpt[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) st[kb] = dpt[kb] = (f32x16){};
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        st[kb] = mfma(lds_b128(kt + koff_l + kb * 32 * RSX + ds * 32), qf[ds], st[kb]);
        dpt[kb] = mfma(lds_b128(vt + voff_l + kb * 32 * RSR + ds * 32), dof[ds], dpt[kb]);
      }
    if (j0 + BC - 1 > kfull_w) {
      // keys past the row's last visible one (and past Nk) get P = 0
      const int klim = CAUSAL ? min(Nk, query + off + 1) : Nk;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int kmax = klim - 1 - j0 - kb * 32 - (lane >> 5) * 4;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if ((i >> 2) * 8 + (i & 3) > kmax) st[kb][i] = NEG_INF;
      }
    }
    u32x4 dsp[PS];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][i], c, -L2));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][i + 1], c, -L2));
        dsp[kb * 2 + i / 8][(i % 8) / 2] = pack_bf16(p0 * (dpt[kb][i] - Drow), p1 * (dpt[kb][i + 1] - Drow));
      }
#pragma unroll
    for (int ps = 0; ps < PS; ++ps)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        dq[db] = mfma(v_frag_p<RSX>(kt + toff_l, ps, db), __builtin_bit_cast(bf16x8, dsp[ps]), dq[db]);
  };

  // double-buffered key tiles: iteration j waits for tile j, then starts the
  // copy of tile j + 1 into the slot tile j - 1 used
  auto iteration = [&](int j, auto par) {
    using other = std::integral_constant<int, 1 - decltype(par)::value>;
    vm_wait<0>();
    __syncthreads();
    if (j + 1 < nt) issue(j + 1, other{});
    if (j < ntw) compute(j, par);
  };
  if (nt > 0) issue(0, P0{});
  for (int j = 0; j < nt; j += 2) {
    iteration(j, P0{});
    if (j + 1 < nt) iteration(j + 1, P1{});
  }
  vm_wait<0>();

  if (!live || query >= Nq) return;
  const size_t orow = qoff + (size_t)query * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      bf16x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = (__bf16)(dq[db][i4 * 4 + e] * scale);
      *(bf16x4*)(dQ + orow + db * 32 + i4 * 8 + (lane >> 5) * 4) = r;
    }
}

// One workgroup per work item.
template <int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1)))
void fa_bwd_dq_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                      const __bf16* __restrict__ O, const __bf16* __restrict__ dO, const float* __restrict__ LSE,
                      float* __restrict__ LD, __bf16* __restrict__ dQ, fa_plan_t p, float c, float scale) {
  bwd_dq_item<D, CAUSAL, NW>(Q, K, V, O, dO, LSE, LD, dQ, p, c, scale, blockIdx.x);
}

// The kernels that hold a whole CU per workgroup (8 waves at d = 128, 4 at
// d = 256) as the forward kernel's persistent grid (fa_persistent_item),
// for plans with more items than CUs.  A kernel of its own, so that the
// one-item kernel keeps its code where it is used.
template <int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1)))
void fa_bwd_dq_persistent_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                 const __bf16* __restrict__ V, const __bf16* __restrict__ O,
                                 const __bf16* __restrict__ dO, const float* __restrict__ LSE, float* __restrict__ LD,
                                 __bf16* __restrict__ dQ, fa_plan_t p, float c, float scale) {
  for (unsigned r = 0;; ++r) {
    const unsigned id = fa_persistent_item(gridDim.x, p.nwg, blockIdx.x, r);
    if (id == ~0u) break;
    if (r > 0) __syncthreads();  // every wave is done with the last item's LDS
    bwd_dq_item<D, CAUSAL, NW>(Q, K, V, O, dO, LSE, LD, dQ, p, c, scale, id);
  }
}
#define FA_INST_DQ_P(DD, CC, NN)                                                                               \
  template __global__ void fa_bwd_dq_persistent_kernel<DD, CC, NN>(                                            \
      const __bf16* __restrict__, const __bf16* __restrict__, const __bf16* __restrict__, const __bf16* __restrict__, \
      const __bf16* __restrict__, const float* __restrict__, float* __restrict__, __bf16* __restrict__, fa_plan_t, \
      float, float);
FA_INST_DQ_P(128, false, 8)
FA_INST_DQ_P(128, true, 8)
FA_INST_DQ_P(256, false, 4)
FA_INST_DQ_P(256, true, 4)
FA_INST_DQ_P(128, true, 4)
#undef FA_INST_DQ_P

// ---------------------------------------------------------------- dK, dV
// Wave state: K and V rows of KBW blocks of 32 keys as B operands (lane: key
// lane % 32, 8 consecutive columns per k-step); dK^T, dV^T accumulators
// (d x 32 per key block).  Per query tile (64 rows of one query head, staged
// in LDS with their L2 = LSE log2(e) and D values), per 32-row half:
//   S  = Q K^T   (A = Q rows from LDS)         dP = dO V^T  (A = dO rows)
//   P  = 2^(S c - L2), dS = P o (dP - D), packed to bf16 in place
//   dV^T += dO^T P,  dK^T += Q^T dS  (A = dO^T, Q^T: transposed LDS reads in
//   the row order of the S accumulator)
// The query tiles are visited last tile first, head-minor: all workgroups of
// one key/value head then read the same query tiles at about the same time,
// from L2.
//
// One work item (fa_kv_decode of id) per call; a persistent workgroup calls
// it once per item, with a barrier in between (LDS is reused).
template <int D, bool CAUSAL, int NW, int KBW>
__device__ __forceinline__ void bwd_dkdv_item(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                              const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                                              const float* __restrict__ LD, __bf16* __restrict__ dK,
                                              __bf16* __restrict__ dV, float* __restrict__ PART,
                                              const fa_kvplan_t& p, float c, float scale, unsigned id) {
  using C = BwdCfg<D>;
  constexpr int DS = C::DS, DB = C::DB, RSX = C::RSX;
  constexpr int KPW = 32 * KBW;
  using CopyQ = CopyPlan<D, NW, C::SPR_X, true>;
  __shared__ __attribute__((aligned(1024))) char lq0_[C::TILE_X];
  __shared__ __attribute__((aligned(1024))) char lq1_[C::TILE_X];
  __shared__ __attribute__((aligned(1024))) char lo0_[C::TILE_X];
  __shared__ __attribute__((aligned(1024))) char lo1_[C::TILE_X];
  // d = 128: the V rows of the workgroup's keys are staged in LDS once (whole
  // tiles of 64 rows) and the V fragments of dP = dO V^T are read from there,
  // which leaves the registers they would take to the compiler for loads in
  // flight.  At d = 256 there is no LDS room; at d = 64 no register pressure.
  constexpr bool VLDS = (D == 128);
  constexpr int RSR = C::RSR;
  constexpr int VT = (NW * KPW + BC - 1) / BC;  // tiles of V rows
  __shared__ __attribute__((aligned(1024))) char lvr_[VLDS ? VT * C::TILE_R : 16];
  __shared__ __attribute__((aligned(1024))) char ll0_[1024];
  __shared__ __attribute__((aligned(1024))) char ll1_[1024];
  __shared__ __attribute__((aligned(1024))) char lsp_[1024];
  auto qslot = [&](auto par) { return (LDS_AS char*)(decltype(par)::value == 0 ? lq0_ : lq1_); };
  auto oslot = [&](auto par) { return (LDS_AS char*)(decltype(par)::value == 0 ? lo0_ : lo1_); };
  auto lslot = [&](auto par) { return (LDS_AS char*)(decltype(par)::value == 0 ? ll0_ : ll1_); };
  LDS_AS char* const spare = (LDS_AS char*)lsp_;

  const fa_kvwork_t w = fa_kv_decode(p, id);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int k0w = w.k0 + wave * KPW;
  const int Nq = p.Nq, Nk = p.Nk, off = Nk - Nq, G = p.G;
  // the workgroup's query heads: hps heads of part w.hs of the group
  const int HP = p.hps, h0 = w.hs * p.hps;
  const size_t kvoff = (size_t)(w.b * p.Hkv + w.hkv) * Nk * D;
  const bool has_keys = k0w < Nk;

  bf16x8 kf[KBW][DS], vf[VLDS ? 1 : KBW][VLDS ? 1 : DS];
#pragma unroll
  for (int kb = 0; kb < KBW; ++kb) {
    const int key = k0w + kb * 32 + (lane & 31);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const size_t e0 = kvoff + (size_t)key * D + ds * 16 + h * 8;
      kf[kb][ds] = key < Nk ? *(const bf16x8*)(K + e0) : (bf16x8){};
      if constexpr (!VLDS) vf[kb][ds] = key < Nk ? *(const bf16x8*)(V + e0) : (bf16x8){};
    }
  }
  if constexpr (VLDS) {
    // copied like the query tiles (rows past Nk read as zero); they land
    // before the barrier of the first iteration
    using CopyV = CopyPlan<D, NW, C::SPR_R>;
    CopyV cv;
    cv.init(wave, lane);
    const __amdgpu_buffer_rsrc_t vres = CopyV::rsrc(V + kvoff, Nk);
#pragma unroll
    for (int t = 0; t < VT; ++t)
      cv.issue_all(vres, (w.k0 + t * BC) * (D * 2), (LDS_AS char*)lvr_ + t * C::TILE_R, (LDS_AS char*)lsp_, wave);
  }
  LDS_AS const char* const vrow = (LDS_AS const char*)lvr_ + wave * KPW * RSR + k_lane_off<RSR>(lane);
  f32x16 dk[KBW][DB], dv[KBW][DB];
#pragma unroll
  for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
    for (int db = 0; db < DB; ++db) dk[kb][db] = dv[kb][db] = (f32x16){};

  int first, ntq;
  fa_kv_query_tiles(p, w.k0, BC, first, ntq);
  // iterations: query tiles ntq - 1 down to first, the HP heads of the
  // workgroup innermost; (t_c, h_c) is the tile and head of the iteration
  // computed
  const int total = (ntq - first) * HP;
  int t_c = ntq - 1, h_c = 0;

  const int qoff_l = k_lane_off_p<RSX>(lane), toff_l = v_lane_off_p<RSX>(lane);
  CopyQ cp;
  cp.init(wave, lane);
  auto issue = [&](int t, int hh, auto par) {
    const int hq = w.hkv * G + h0 + hh;
    const size_t rb = (size_t)(w.b * p.Hq + hq) * Nq;
    const __amdgpu_buffer_rsrc_t rq = CopyQ::rsrc(Q + rb * D, Nq), ro = CopyQ::rsrc(dO + rb * D, Nq);
    cp.issue_all(rq, t * (BC * D * 2), qslot(par), spare, wave);
    cp.issue_all(ro, t * (BC * D * 2), oslot(par), spare, wave);
    if (wave == 0) {
      // (L2, D) of the tile's 64 rows: 512 bytes from lanes 0 .. 31 (lanes
      // 32 .. 63 fill the unused second half of the 1 KB slot)
      const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc((void*)(LD + rb * 2), (short)0, Nq * 8, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (LDS_AS void*)lslot(par), 16, lane * 16, t * (BC * 8), 0, 0);
    }
  };

  auto compute = [&](int q0, auto par) {
    LDS_AS const char* qt = qslot(par);
    LDS_AS const char* ot = oslot(par);
    LDS_AS const char* lt = lslot(par);
    // the two 32-row halves one after the other (overlapping them would need
    // a second set of score registers)
#pragma unroll 1
    for (int qb = 0; qb < 2; ++qb) {
      const int qb0 = q0 + qb * 32;
      // wave-uniform skips: rows past Nq, or no row of the half sees the
      // wave's first key
      if (qb0 >= Nq || (CAUSAL && qb0 + 31 + off < k0w)) continue;
      LDS_AS const char* qh = qt + qb * 32 * RSX;
      LDS_AS const char* oh = ot + qb * 32 * RSX;
      f32x16 s[KBW], dp[KBW];
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) s[kb] = dp[kb] = (f32x16){};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const bf16x8 a = lds_b128(qh + qoff_l + ds * 32);
        const bf16x8 b = lds_b128(oh + qoff_l + ds * 32);
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) {
          s[kb] = mfma(a, kf[kb][ds], s[kb]);
          if constexpr (VLDS) dp[kb] = mfma(b, lds_b128(vrow + kb * 32 * RSR + ds * 32), dp[kb]);
          else dp[kb] = mfma(b, vf[kb][ds], dp[kb]);
        }
      }
      // causal, halves that cross the diagonal only (a wave-uniform branch):
      // scores of keys past a row's last visible key become -inf, so P = 0
      if (CAUSAL && k0w + KPW - 1 > qb0 + off) {
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) {
          // row qb0 + 8g + 4h + r misses this lane's key iff 8g + r < lim
          const int lim = k0w + kb * 32 + (lane & 31) - off - qb0 - 4 * h;
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if ((i >> 2) * 8 + (i & 3) < lim) s[kb][i] = NEG_INF;
        }
      }
      // P and dS of the half, packed to bf16
      u32x4 pp[KBW][2], dsp[KBW][2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // (L2, D) of the lane's rows qb*32 + 8g + 4h + r, r = 0 .. 3
        LDS_AS const f32x4* src = (LDS_AS const f32x4*)(lt + (qb * 32 + 8 * g + 4 * h) * 8);
        const f32x4 la = src[0], lb = src[1];
        const float l2v[4] = {la[0], la[2], lb[0], lb[2]}, ddv[4] = {la[1], la[3], lb[1], lb[3]};
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) {
#pragma unroll
          for (int r = 0; r < 4; r += 2) {
            float pr[2], dsv[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              pr[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][4 * g + r + u], c, -l2v[r + u]));
              dsv[u] = pr[u] * (dp[kb][4 * g + r + u] - ddv[r + u]);
            }
            pp[kb][g / 2][2 * (g % 2) + r / 2] = pack_bf16(pr[0], pr[1]);
            dsp[kb][g / 2][2 * (g % 2) + r / 2] = pack_bf16(dsv[0], dsv[1]);
          }
        }
      }
#pragma unroll
      for (int ps = 0; ps < 2; ++ps)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 a = v_frag_p<RSX>(oh + toff_l, ps, db);
#pragma unroll
          for (int kb = 0; kb < KBW; ++kb) dv[kb][db] = mfma(a, __builtin_bit_cast(bf16x8, pp[kb][ps]), dv[kb][db]);
        }
#pragma unroll
      for (int ps = 0; ps < 2; ++ps)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 a = v_frag_p<RSX>(qh + toff_l, ps, db);
#pragma unroll
          for (int kb = 0; kb < KBW; ++kb) dk[kb][db] = mfma(a, __builtin_bit_cast(bf16x8, dsp[kb][ps]), dk[kb][db]);
        }
    }
  };

  auto iteration = [&](int it, auto par) {
    using other = std::integral_constant<int, 1 - decltype(par)::value>;
    vm_wait<0>();
    __syncthreads();
    const int h_n = h_c + 1 == HP ? 0 : h_c + 1;
    const int t_n = h_c + 1 == HP ? t_c - 1 : t_c;
    if (it + 1 < total) issue(t_n, h_n, other{});
    const int q0 = t_c * BC;
    if (has_keys && (!CAUSAL || q0 + BC - 1 + off >= k0w)) compute(q0, par);
    t_c = t_n;
    h_c = h_n;
  };
  if (total > 0) issue(ntq - 1, 0, P0{});
  for (int it = 0; it < total; it += 2) {
    iteration(it, P0{});
    if (it + 1 < total) iteration(it + 1, P1{});
  }
  vm_wait<0>();

  // with the heads split into parts, this part's sums (dK already scaled)
  // go to its fp32 slice of the workspace; fa_bwd_reduce_kernel adds them
  const size_t part_elems = (size_t)p.B * p.Hkv * Nk * D;
#pragma unroll
  for (int kb = 0; kb < KBW; ++kb) {
    const int key = k0w + kb * 32 + (lane & 31);
    if (key >= Nk) continue;
    const size_t krow = kvoff + (size_t)key * D;
    if (p.hsplit > 1) {
      float* pk = PART + (size_t)w.hs * part_elems + krow;
      float* pv = PART + (size_t)(p.hsplit + w.hs) * part_elems + krow;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = db * 32 + i4 * 8 + h * 4;
          f32x4 rk, rv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            rk[e] = dk[kb][db][i4 * 4 + e] * scale;
            rv[e] = dv[kb][db][i4 * 4 + e];
          }
          *(f32x4*)(pk + d0) = rk;
          *(f32x4*)(pv + d0) = rv;
        }
      continue;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = db * 32 + i4 * 8 + h * 4;
        bf16x4 rk, rv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          rk[e] = (__bf16)(dk[kb][db][i4 * 4 + e] * scale);
          rv[e] = (__bf16)dv[kb][db][i4 * 4 + e];
        }
        *(bf16x4*)(dK + krow + d0) = rk;
        *(bf16x4*)(dV + krow + d0) = rv;
      }
  }
}

// One workgroup per key block (and head part).
template <int D, bool CAUSAL, int NW, int KBW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1)))
void fa_bwd_dkdv_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                        const __bf16* __restrict__ dO, const float* __restrict__ LD, __bf16* __restrict__ dK,
                        __bf16* __restrict__ dV, float* __restrict__ PART, fa_kvplan_t p, float c, float scale) {
  bwd_dkdv_item<D, CAUSAL, NW, KBW>(Q, K, V, dO, LD, dK, dV, PART, p, c, scale, blockIdx.x);
}

// The dK/dV kernels as a persistent grid of fewer workgroups than items
// (fa_persistent_item over the key-block order): the snake gives every
// workgroup heavy and light causal key blocks alike.  Forms (launch_bwd_dkdv
// picks them up to Nq = 4096 with at least two items per workgroup), with
// the workgroups each CU holds: 8 waves at d = 128 (one per CU), 4 waves at
// d = 128, 256 and 64 (one per CU), 2 waves at d = 64, causal only (two per
// CU; non-causal 2-wave d = 64 plans never reach two items per workgroup).
// A kernel of its own: the loop around the item slows the one-item kernel's
// inner loop by 3-5 % where that is kept (Nq > 4096).
template <int D, bool CAUSAL, int NW, int KBW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1)))
void fa_bwd_dkdv_persistent_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                   const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                                   const float* __restrict__ LD, __bf16* __restrict__ dK, __bf16* __restrict__ dV,
                                   float* __restrict__ PART, fa_kvplan_t p, float c, float scale) {
  for (unsigned r = 0;; ++r) {
    const unsigned id = fa_persistent_item(gridDim.x, p.nwg, blockIdx.x, r);
    if (id == ~0u) break;
    if (r > 0) __syncthreads();  // every wave is done with the last item's LDS
    bwd_dkdv_item<D, CAUSAL, NW, KBW>(Q, K, V, dO, LD, dK, dV, PART, p, c, scale, id);
  }
}
#define FA_INST_DKDV_P(DD, CC, NN, KK)                                                                         \
  template __global__ void fa_bwd_dkdv_persistent_kernel<DD, CC, NN, KK>(                                      \
      const __bf16* __restrict__, const __bf16* __restrict__, const __bf16* __restrict__, const __bf16* __restrict__, \
      const float* __restrict__, __bf16* __restrict__, __bf16* __restrict__, float* __restrict__, fa_kvplan_t,   \
      float, float);
FA_INST_DKDV_P(128, false, 8, 1)
FA_INST_DKDV_P(128, true, 8, 1)
FA_INST_DKDV_P(256, false, 4, 1)
FA_INST_DKDV_P(256, true, 4, 1)
FA_INST_DKDV_P(64, false, 4, 2)
FA_INST_DKDV_P(64, true, 4, 2)
FA_INST_DKDV_P(64, true, 2, 2)
FA_INST_DKDV_P(128, false, 4, 1)
FA_INST_DKDV_P(128, true, 4, 1)
#undef FA_INST_DKDV_P

// ---------------------------------------------------------------- launchers
// dK and dV from the head parts' partial sums: for every element, the sum
// over the parts of the fp32 partials (dK's already scaled), rounded to bf16.
// PART holds [parts][B][Hkv][Nk][d] for dK, then the same for dV; n4 is the
// number of 4-element groups of one tensor.  A grid-stride loop over both.
__global__ __launch_bounds__(256) void fa_bwd_reduce_kernel(const float* __restrict__ PART, int parts, long long n4,
                                                            __bf16* __restrict__ dK, __bf16* __restrict__ dV) {
  const long long n = 4 * n4;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < 2 * n4; i += (long long)gridDim.x * 256) {
    const int tensor = i < n4 ? 0 : 1;
    const long long j = i - tensor * n4;
    const float* src = PART + (size_t)tensor * parts * n + 4 * j;
    f32x4 acc = *(const f32x4*)src;
    for (int sp = 1; sp < parts; ++sp) acc += *(const f32x4*)(src + (size_t)sp * n);
    bf16x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = (__bf16)acc[e];
    *(bf16x4*)((tensor == 0 ? dK : dV) + 4 * j) = r;
  }
}

#define FA_INST_DQ(DD, CC, NN)                                                                                  \
  template __global__ void fa_bwd_dq_kernel<DD, CC, NN>(                                                       \
      const __bf16* __restrict__, const __bf16* __restrict__, const __bf16* __restrict__, const __bf16* __restrict__, \
      const __bf16* __restrict__, const float* __restrict__, float* __restrict__, __bf16* __restrict__, fa_plan_t,  \
      float, float);
// (head dim, causal, waves per workgroup)
#define FA_DQ_VARIANTS(X)                                                                                    \
  X(64, false, 1) X(64, false, 2) X(64, false, 4) X(64, false, 8) X(64, true, 1) X(64, true, 2)                \
  X(64, true, 4) X(64, true, 8) X(128, false, 1) X(128, false, 2) X(128, false, 4) X(128, false, 8)            \
  X(128, true, 1) X(128, true, 2) X(128, true, 4) X(128, true, 8) X(256, false, 1) X(256, false, 2)            \
  X(256, false, 4) X(256, true, 1) X(256, true, 2) X(256, true, 4)
FA_DQ_VARIANTS(FA_INST_DQ)

#define FA_INST_DKDV(DD, CC, NN, KK)                                                                           \
  template __global__ void fa_bwd_dkdv_kernel<DD, CC, NN, KK>(                                                \
      const __bf16* __restrict__, const __bf16* __restrict__, const __bf16* __restrict__, const __bf16* __restrict__, \
      const float* __restrict__, __bf16* __restrict__, __bf16* __restrict__, float* __restrict__, fa_kvplan_t,   \
      float, float);
// (head dim, causal, waves per workgroup, 32-key blocks per wave)
#define FA_DKDV_VARIANTS(X)                                                                                  \
  X(64, false, 1, 2) X(64, false, 2, 2) X(64, false, 4, 2) X(64, true, 1, 2) X(64, true, 2, 2)                 \
  X(64, true, 4, 2) X(128, false, 1, 1) X(128, false, 2, 1) X(128, false, 4, 1) X(128, false, 8, 1)            \
  X(128, true, 1, 1) X(128, true, 2, 1) X(128, true, 4, 1) X(128, true, 8, 1) X(256, false, 1, 1)              \
  X(256, false, 2, 1) X(256, false, 4, 1) X(256, true, 1, 1) X(256, true, 2, 1) X(256, true, 4, 1)
FA_DKDV_VARIANTS(FA_INST_DKDV)

int bwd_keys_per_wave(int d) { return d == 64 ? 64 : 32; }

int bwd_dkdv_max_waves(int d) { return d == 64 ? 4 : d == 128 ? 8 : 4; }

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, void* dq, float* ld, const fa_plan_t& pq, int d, float c, float scale,
                         hipStream_t stream) {
  // persistent: the 8-wave d = 128 kernel always (configuration-3 backward
  // +0.4 %, N2048 +1.6 %), the 4-wave d = 256 one up to Nq = 4096 (causal
  // N1024-2048 +22-29 % with the dK/dV grid; at N8192 2 % slower)
  // (the causal 4-wave d = 128 kernel fits two workgroups per CU and runs
  // two per CU under the d = 256 rule)
  const bool two = d == 128 && pq.nw == 4 && pq.causal && pq.Nq <= 4096;
  const bool persist = (d == 128 && pq.nw == 8) || (d == 256 && pq.nw == 4 && pq.Nq <= 4096) || two;
  const unsigned grid = persist ? persistent_grid(pq.nwg, two ? 2 : 1) : 0;
  if (grid > 0 && (long long)grid < pq.nwg) {
#define FA_DQ_P(DD, CC, NN)                                                                                    \
  hipLaunchKernelGGL((fa_bwd_dq_persistent_kernel<DD, CC, NN>), dim3(grid), dim3(64 * NN), 0, stream,            \
                     (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)o, (const __bf16*)dout, \
                     lse, ld, (__bf16*)dq, pq, c, scale)
    if (two) {
      FA_DQ_P(128, true, 4);
    } else if (d == 128) {
      if (pq.causal) FA_DQ_P(128, true, 8);
      else FA_DQ_P(128, false, 8);
    } else {
      if (pq.causal) FA_DQ_P(256, true, 4);
      else FA_DQ_P(256, false, 4);
    }
#undef FA_DQ_P
    return hipGetLastError();
  }
#define FA_CASE_DQ(DD, CC, NN)                                                                             \
  if (d == DD && (pq.causal != 0) == CC && pq.nw == NN) {                                                   \
    hipLaunchKernelGGL((fa_bwd_dq_kernel<DD, CC, NN>), dim3((unsigned)pq.nwg), dim3(64 * NN), 0, stream,       \
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)o,                  \
                       (const __bf16*)dout, lse, ld, (__bf16*)dq, pq, c, scale);                              \
    return hipGetLastError();                                                                               \
  }
  FA_DQ_VARIANTS(FA_CASE_DQ)
#undef FA_CASE_DQ
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dv,
                           const float* ld, float* part, const fa_kvplan_t& pk, int d, float c, float scale,
                           hipStream_t stream) {
  if (pk.hsplit > 1 && part == nullptr) return hipErrorInvalidValue;
  hipError_t e = hipErrorInvalidValue;
  // persistent grids up to 64 query tiles per key block (Nq <= 4096) and
  // with at least two items per workgroup: measured 3-29 % faster there
  // (d = 64, 128, 256; MHA and GQA; N 1024-4096); longer sequences and
  // partial second rounds keep one workgroup per item
  // workgroups per CU of the kernels with a persistent form: one for 8 waves
  // at d = 128 (two waves per SIMD) and 4 waves at d = 128, 256 and 64 (one
  // wave per SIMD), two for 2 waves at d = 64
  const int per_cu = ((d == 128 && (pk.nw == 8 || pk.nw == 4)) || (d == 256 && pk.nw == 4) || (d == 64 && pk.nw == 4))
                         ? 1
                     : (d == 64 && pk.nw == 2 && pk.causal) ? 2 : 0;
  const unsigned grid = (per_cu > 0 && pk.Nq <= 4096) ? persistent_grid(pk.nwg, per_cu) : 0;
  if (grid > 0 && 2LL * grid <= pk.nwg) {
#define FA_DKDV_P(DD, CC, NN, KK)                                                                              \
  hipLaunchKernelGGL((fa_bwd_dkdv_persistent_kernel<DD, CC, NN, KK>), dim3(grid), dim3(64 * NN), 0, stream,      \
                     (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)dout, ld, (__bf16*)dk, \
                     (__bf16*)dv, part, pk, c, scale)
    if (d == 128 && pk.nw == 8) {
      if (pk.causal) FA_DKDV_P(128, true, 8, 1);
      else FA_DKDV_P(128, false, 8, 1);
    } else if (d == 128) {
      if (pk.causal) FA_DKDV_P(128, true, 4, 1);
      else FA_DKDV_P(128, false, 4, 1);
    } else if (d == 256) {
      if (pk.causal) FA_DKDV_P(256, true, 4, 1);
      else FA_DKDV_P(256, false, 4, 1);
    } else if (pk.nw == 4) {
      if (pk.causal) FA_DKDV_P(64, true, 4, 2);
      else FA_DKDV_P(64, false, 4, 2);
    } else {
      FA_DKDV_P(64, true, 2, 2);  // per_cu > 0 at d = 64 with 2 waves only if causal
    }
#undef FA_DKDV_P
    e = hipGetLastError();
  } else
#define FA_CASE_DKDV(DD, CC, NN, KK)                                                                        \
  if (d == DD && (pk.causal != 0) == CC && pk.nw == NN && pk.kpw == 32 * KK) {                              \
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<DD, CC, NN, KK>), dim3((unsigned)pk.nwg), dim3(64 * NN), 0, stream, \
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)dout, ld,          \
                       (__bf16*)dk, (__bf16*)dv, part, pk, c, scale);                                         \
    e = hipGetLastError();                                                                                  \
  } else
  FA_DKDV_VARIANTS(FA_CASE_DKDV) {}
#undef FA_CASE_DKDV
  if (e != hipSuccess || pk.hsplit == 1) return e;
  const long long n4 = (long long)pk.B * pk.Hkv * pk.Nk * d / 4;  // float4 groups per tensor
  const long long blocks = (2 * n4 + 255) / 256;
  hipLaunchKernelGGL(fa_bwd_reduce_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, stream,
                     (const float*)part, pk.hsplit, n4, (__bf16*)dk, (__bf16*)dv);
  return hipGetLastError();
}

}  // namespace fa

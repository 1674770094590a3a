// fa_fwd_fp8.hip -- fused exact-attention forward kernel on e4m3 operands
// for gfx950 (MI355X).
//
// The FP8 form of the fused forward pass ("FlashAttention-3 — 闪电注意力-3",
// sections on Hopper's FP8 support and on low precision): both matrix
// products run on 8-bit floating point, whose dense peak is twice that of
// bf16, with fp32 accumulation.  The operands come from fa_fp8_prepare (Q
// and K rotated by a signed Hadamard matrix and quantised with one scale per
// tensor, V quantised and stored transposed).  The structure is that of the
// bf16 kernel: 32 query rows per wave with their Q codes resident in VGPRs,
// K and V^T tiles of 64 keys copied HBM -> LDS with bounds-checked buffer
// loads, double buffered; scores transposed (S^T = K Q^T) so that a lane
// holds the scores of one query; the online softmax with the output
// rescaled only when a row maximum grows by more than TAU; causal tiles
// above the diagonal skipped.
#include <hip/hip_runtime.h>
#include <stdint.h>

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
// Descales: the score scale folds s_q s_k into c, the epilogue multiplies O
// by s_v / l.  P (at most 2^TAU = 256 < 448) is quantised unscaled.
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
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
  __device__ __forceinline__ void issue_all(const __amdgpu_buffer_rsrc_t& rs, int soff, LDS_AS char* tile,
                                            LDS_AS char* spare, int wave) const {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int ins = i * NW + wave;
      LDS_AS char* dst = (INS % NW == 0 || ins < INS) ? tile + ins * 1024 : spare;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)dst, 16, goff[i], soff, 0, 0);
    }
  }
};

template <int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1)))
void fa_fwd_fp8_kernel(const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ K8,
                       const uint8_t* __restrict__ V8T, const float* __restrict__ descale,
                       __bf16* __restrict__ O, float* __restrict__ LSE, fa_plan_t p, float c0) {
  constexpr int KB = BC / 32;      // 32-key blocks per tile
  constexpr int KS = D / 64;       // k-steps of S^T
  constexpr int DB = D / 32;       // 32-row blocks of O^T
  constexpr int NMF = KB * KS;     // S^T MFMAs per tile
  constexpr int SPS = KB * 16 / NMF;  // exponentials per S^T MFMA
  constexpr int RSK = D + 16;      // K8 LDS row stride (conflict-free for 16 consecutive keys)
  constexpr int RSV = 80;          // V8^T LDS row stride: 64 keys + 16 bytes
  constexpr int KTILE = BC * RSK, VTILE = D * RSV;
  using KCopy = TileCopy<BC, D / 16, D / 16 + 1, NW>;
  using VCopy = TileCopy<D, 4, 5, NW>;
  constexpr int MIK = KCopy::MI, MIV = VCopy::MI;
  __shared__ __attribute__((aligned(1024))) char smem_[2 * KTILE + 2 * VTILE + 1024];
  LDS_AS char* const smem = (LDS_AS char*)smem_;
  LDS_AS char* const spare = smem + 2 * KTILE + 2 * VTILE;

  const fa_work_t w = fa_decode(p, blockIdx.x);
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
  const int ntw = (live && klast_w >= 0) ? min(nt, klast_w / BC + 1) : 0;
  const float sq = descale[0], sk = descale[1], sv = descale[2];
  const float c = c0 * sq * sk;

  const size_t qoff = (size_t)(w.b * p.Hq + hq) * Nq * D;
  const size_t koff = (size_t)(w.b * p.Hkv + w.hkv) * Nk * D;
  const size_t voff = (size_t)(w.b * p.Hkv + w.hkv) * D * Nkp;

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
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = (f32x16){};
  float m_ref = NEG_INF, m_run = NEG_INF, lsum = 0.f;

  const int koff_l = (lane & 31) * RSK + (lane >> 5) * 32;
  const int voff_l = (lane & 31) * RSV + (lane >> 5) * 32;
  KCopy kc;
  VCopy vc;
  kc.init(wave, lane, D);
  vc.init(wave, lane, Nkp);
  const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc((void*)(K8 + koff), (short)0, Nk * D, 0x00020000);
  const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc((void*)(V8T + voff), (short)0, D * Nkp, 0x00020000);
  auto opaque = [](int x) {
    asm volatile("" : "+s"(x));
    return x;
  };
  auto kslot = [&](int t) { return smem + (t & 1) * KTILE; };
  auto vslot = [&](int t) { return smem + 2 * KTILE + (t & 1) * VTILE; };
  auto copy_k = [&](int t) {
    kc.issue_all(kres, t < nt ? t * BC * D : Nk * D, smem + opaque((t & 1) * KTILE), spare, wave);
  };
  auto copy_v = [&](int t) {
    vc.issue_all(vres, t < nt ? t * BC : D * Nkp, smem + opaque(2 * KTILE + (t & 1) * VTILE), spare, wave);
  };

  // prologue: K_0, V_0, K_1 complete; S_0
  copy_k(0);
  copy_k(1);
  copy_v(0);
  vm_wait<0>();
  __syncthreads();
  f32x16 sa[KB], sb[KB];
  auto scores = [&](f32x16 (&sv_)[KB], LDS_AS const char* kt) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sv_[kb] = (f32x16){};
#pragma unroll
    for (int t = 0; t < NMF; ++t) {
      const int ks = t / KB, kb = t % KB;
      sv_[kb] = mfma_fp8(lds_b256(kt + koff_l + kb * 32 * RSK + ks * 64), qf[ks], sv_[kb]);
    }
  };
  if (ntw > 0) scores(sa, kslot(0));

  auto step = [&](int j, f32x16 (&s)[KB], f32x16 (&sn)[KB]) {
    const int j0 = j * BC;
    vm_wait<0>();
    __syncthreads();
    if (j + 2 < nt) copy_k(j + 2);
    if (j + 1 < nt) copy_v(j + 1);
    if (j >= ntw) return;
    LDS_AS const char* knext = kslot(j + 1) + koff_l;
    LDS_AS const char* vlane = vslot(j) + voff_l;
    i32x8 kbuf = lds_b256(knext);

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

    float mu = (m_ref == NEG_INF) ? 0.f : m_ref;
    float part0 = 0.f, part1 = 0.f;
    float pfl[KB * 16];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sn[kb] = (f32x16){};
#pragma unroll
    for (int t = 0; t < NMF; ++t) {
      const int ks = t / KB, kb = t % KB;
      const i32x8 kf = kbuf;
      if (t + 1 < NMF) kbuf = lds_b256(knext + ((t + 1) % KB) * 32 * RSK + ((t + 1) / KB) * 64);
      sn[kb] = mfma_fp8(kf, qf[ks], sn[kb]);
#pragma unroll
      for (int u = 0; u < SPS; ++u) {
        const int sc = t * SPS + u;
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sc / 16][sc % 16], c, -mu));
        if (sc & 1) part1 += pv;
        else part0 += pv;
        pfl[sc] = pv;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    float part = part0 + part1;
    if (__ballot(!(part <= TAU_EXP2) || m_ref == NEG_INF)) {
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
      mu = (m_ref == NEG_INF) ? 0.f : m_ref;
      part = 0.f;
#pragma unroll
      for (int sc = 0; sc < KB * 16; ++sc) {
        pfl[sc] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sc / 16][sc % 16], c, -mu));
        part += pfl[sc];
      }
    }
    lsum += part;
    // P -> e4m3, byte j = score j (block j/16, register j%16)
    i32x8 p8;
#pragma unroll
    for (int wd = 0; wd < 8; ++wd) {
      int v = __builtin_amdgcn_cvt_pk_fp8_f32(pfl[4 * wd], pfl[4 * wd + 1], 0, false);
      p8[wd] = __builtin_amdgcn_cvt_pk_fp8_f32(pfl[4 * wd + 2], pfl[4 * wd + 3], v, true);
    }
    // O^T += V^T P^T: one MFMA per 32-row block of d covers the 64 keys
    i32x8 vbuf = lds_b256(vlane);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const i32x8 vf = vbuf;
      if (db + 1 < DB) vbuf = lds_b256(vlane + (db + 1) * 32 * RSV);
      o[db] = mfma_fp8(vf, p8, o[db]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int j = 0; j < nt; j += 2) {
    step(j, sa, sb);
    if (j + 1 < nt) step(j + 1, sb, sa);
  }
  (void)vslot;
  // the last copies (zeros past the final tile) land before the workgroup's
  // LDS can pass to another workgroup
  vm_wait<0>();

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

// ---------------------------------------------------------------- launcher
#define FA_INST_FP8(DD, CC, NN)                                                                              \
  template __global__ void fa_fwd_fp8_kernel<DD, CC, NN>(const uint8_t* __restrict__, const uint8_t* __restrict__, \
                                                         const uint8_t* __restrict__, const float* __restrict__,   \
                                                         __bf16* __restrict__, float* __restrict__, fa_plan_t, float);
#define FA_FP8_VARIANTS(X)                                                                                  \
  X(64, false, 1) X(64, false, 2) X(64, false, 4) X(64, true, 1) X(64, true, 2) X(64, true, 4)              \
  X(128, false, 1) X(128, false, 2) X(128, false, 4) X(128, true, 1) X(128, true, 2) X(128, true, 4)        \
  X(256, false, 1) X(256, false, 2) X(256, false, 4) X(256, true, 1) X(256, true, 2) X(256, true, 4)
FA_FP8_VARIANTS(FA_INST_FP8)

hipError_t launch_fwd_fp8(const void* q8, const void* k8, const void* v8t, const float* descale, void* o, float* lse,
                          const fa_plan_t& p, int d, float c, hipStream_t stream) {
#define FA_CASE_FP8(DD, CC, NN)                                                                           \
  if (d == DD && (p.causal != 0) == CC && p.nw == NN) {                                                 \
    hipLaunchKernelGGL((fa_fwd_fp8_kernel<DD, CC, NN>), dim3((unsigned)p.nwg), dim3(64 * NN), 0, stream,     \
                       (const uint8_t*)q8, (const uint8_t*)k8, (const uint8_t*)v8t, descale, (__bf16*)o, lse, p, \
                       c);                                                                              \
    return hipGetLastError();                                                                           \
  }
  FA_FP8_VARIANTS(FA_CASE_FP8)
#undef FA_CASE_FP8
  return hipErrorInvalidValue;
}

}  // namespace fa

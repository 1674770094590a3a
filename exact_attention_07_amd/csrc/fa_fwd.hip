// fa_fwd.hip -- fused exact-attention forward kernels for gfx950 (MI355X).
//
// One kernel computes O = softmax(scale * Q K^T) V and LSE for a block of
// query rows without writing scores to memory ("FlashAttention (SV)",
// sections "Tiling och blockbearbetning", "Online-beräkning av Softmax",
// "Sammanslagning av operationer").
//
// Mapping onto CDNA4
// ------------------
// * Each wave owns QPW query rows (two 32-row blocks for d = 64, one for
//   d >= 128) and keeps their Q fragments in VGPRs for the whole pass; at
//   d <= 128 a wave needs at most 256 VGPRs, so two waves share each SIMD and
//   one wave's softmax overlaps the other's matrix products.
// * A workgroup of NW waves (plan.h) streams K/V tiles of BC = 64 keys
//   through LDS.  bf16 tiles are copied HBM -> LDS directly with
//   buffer_load_dwordx4 ... lds (16 B per lane, bounds-checked by the buffer
//   resource so rows past the end read as zero), double buffered, so the copy
//   of tile j+1 overlaps the math on tile j (the asynchronous next-block load
//   of "FlashAttention-3 — 闪电注意力-3", section on minimising memory
//   operations).  LDS rows are padded so that both the row reads of K and the
//   transposed reads of V hit distinct banks with plain "lane base +
//   constant" addresses.
// * Scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16:
//   the accumulator then holds, in each lane, 16 keys of ONE query, so a row
//   maximum is an in-lane max plus one v_permlane32_swap, and the fp32
//   accumulator registers, rounded to bf16, are directly the B operand of
//   O^T += V^T P^T (no LDS round trip for P).  V^T fragments come from LDS
//   with ds_read_b64_tr_b16.
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

#include "fa_kernels.h"
#include "plan.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float TAU = 8.0f;     // rescale threshold, log2 units
constexpr int BC = 64;          // keys per K/V tile
constexpr float NEG_INF = -__builtin_inff();
constexpr float LN2 = 0.693147180559945309f;

template <int D, bool F32>
struct Cfg {
  // query rows per wave: d = 64 keeps 64 rows, d >= 128 keeps 32 so that
  // (d = 128) the whole wave state fits in 256 VGPRs and two waves share a SIMD
  static constexpr int QPW = (D == 64 && !F32) ? 64 : 32;
  static constexpr int WAVES_PER_SIMD = (D <= 128) ? 2 : 1;
  static constexpr int QB = QPW / 32;  // 32-row query blocks per wave
  static constexpr int KB = BC / 32;   // 32-key blocks per tile
  static constexpr int DS = D / 16;    // k-steps of S^T = K Q^T
  static constexpr int DB = D / 32;    // 32-row blocks of O^T
  static constexpr int PS = BC / 16;   // k-steps of O^T += V^T P^T
  // LDS tile: BC rows of D bf16, each row padded by PAD 16-byte slots.  The
  // row stride RS makes both access patterns conflict-free on the 64 banks:
  // 16 lanes reading one 16-byte chunk of 16 consecutive rows (K fragments),
  // and 16 lanes reading a pair of adjacent chunks of 4 consecutive rows (the
  // transposed V reads), while every address stays "lane base + constant".
  static constexpr int CPR = D / 8;                    // data slots per row
  static constexpr int PAD = (D == 64) ? 1 : 3;
  static constexpr int SPR = CPR + PAD;                // slots per LDS row
  static constexpr int RS = SPR * 16;                  // LDS row stride, bytes
  static constexpr int TILE = BC * RS;                 // bytes of one tile
  static constexpr int SLOTS = BC * SPR;
  static constexpr int INS = (SLOTS + 63) / 64;        // 64-lane copy instructions per tile
  static constexpr int STAGES = F32 ? 1 : 2;
  static constexpr int TILES_PER_STAGE = F32 ? 4 : 2;  // K,V (bf16) or Khi,Klo,Vhi,Vlo
  static constexpr int LDS = STAGES * TILES_PER_STAGE * TILE;
};

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Combine a value across the two 32-lane halves (lanes l and l^32 hold the
// same query column of the S^T accumulator).
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8 lds_b128(LDS_AS const char* p) { return *(LDS_AS const bf16x8*)p; }

__device__ __forceinline__ bf16x8 join(i16x4 a, i16x4 b) {
  i16x8 v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Per-lane byte offset of the K fragment (A operand of S^T = K Q^T):
// row lane%32 of the 32-key block, chunk lane/32 of the 16-element k-step.
template <int RS>
__device__ __forceinline__ int k_lane_off(int lane) { return (lane & 31) * RS + (lane >> 5) * 16; }

// Per-lane byte offset of the transposed V read.  The V^T fragment of k-step
// ps and d-block db holds, in element e of lane l, V[ps*16 + (e/4)*8 +
// (l/32)*4 + e%4][db*32 + l%32] (the key order of the S^T accumulator).
// ds_read_b64_tr_b16 gives output lane t of each 16-lane group element c =
// element t%4 of the 8 bytes addressed by lane 4c + t/4 of the group, so lane
// (16g + s) addresses row (g/2)*4 + s/4 (+ ps*16 + 8h), columns
// db*32 + 16(g%2) + 4(s%4) .. +3.
template <int RS>
__device__ __forceinline__ int v_lane_off(int lane) {
  const int g = lane >> 4, s = lane & 15;
  return ((g >> 1) * 4 + (s >> 2)) * RS + (2 * (g & 1) + ((s & 3) >> 1)) * 16 + (s & 1) * 8;
}

template <int RS>
__device__ __forceinline__ bf16x8 v_frag(LDS_AS const char* vlane, int ps, int db) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vlane + (ps * 16) * RS + db * 64));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vlane + (ps * 16 + 8) * RS + db * 64));
  return join(a, b);
}

// HBM -> LDS copy plan of one wave: copy instruction i of the wave (global
// instruction index i*NW + wave) fills LDS bytes [ins*1024, ins*1024 + 1024)
// of the tile, lane t the slot ins*64 + t (BC*SPR is a multiple of 64, so
// the last instruction ends exactly at the end of the tile).  goff is the
// byte offset of the slot's data within the tile's rows in HBM (rows of D
// bf16, contiguous); padding slots get an offset past any buffer range, so
// their load reads zero and writes it into the (never read) padding.
template <int D, int NW>
struct CopyPlan {
  using C = Cfg<D, false>;
  static constexpr int MI = (C::INS + NW - 1) / NW;
  static constexpr unsigned OUT_OF_RANGE = 0x7ffffff0u;
  unsigned goff[MI];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int sl = (i * NW + wave) * 64 + lane;
      const int r = sl / C::SPR, pp = sl % C::SPR;
      goff[i] = pp < C::CPR ? (unsigned)(r * (D * 2) + pp * 16) : OUT_OF_RANGE;
    }
  }
  // Copy BC rows starting at key j0 of a [Nk][D] bf16 matrix; rows >= Nk
  // fall outside the buffer range and read as zero.
  __device__ __forceinline__ void issue(const __bf16* base, int j0, int Nk, LDS_AS char* tile, int wave) const {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(base + (size_t)j0 * D), (short)0, (Nk - j0) * (D * 2), 0x00020000);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      if (i * NW + wave < C::INS)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(tile + (i * NW + wave) * 1024), 16, goff[i], 0,
                                                 0, 0);
    }
  }
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
template <int D>
__device__ __forceinline__ void copy_tile_f32(const float* src, int j0, int Nk, LDS_AS char* tile_hi,
                                              LDS_AS char* tile_lo) {
  using C = Cfg<D, true>;
  for (int sl = threadIdx.x; sl < C::SLOTS; sl += blockDim.x) {
    const int r = sl / C::SPR, pp = sl % C::SPR;
    if (pp >= C::CPR) continue;
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

template <int D, bool CAUSAL, bool F32, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(Cfg<D, F32>::WAVES_PER_SIMD)))
void fa_fwd_kernel(const void* __restrict__ Qp, const void* __restrict__ Kp, const void* __restrict__ Vp,
                   void* __restrict__ Op, float* __restrict__ LSE, fa_plan_t p, float c) {
  using C = Cfg<D, F32>;
  constexpr int QPW = C::QPW, QB = C::QB, KB = C::KB, DS = C::DS, DB = C::DB, PS = C::PS, RS = C::RS;
  __shared__ __attribute__((aligned(1024))) char smem_[C::LDS];
  LDS_AS char* const smem = (LDS_AS char*)smem_;

  const fa_work_t w = fa_decode(p, blockIdx.x);
  // the wave index is uniform across the wave: keep it in an SGPR
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hq = w.hq0 + wave % p.hw;
  const int q0w = w.qpos0 + (wave / p.hw) * QPW;
  const int Nq = p.Nq, Nk = p.Nk;
  const int ntiles = fa_num_kv_tiles(p, w.qpos0, BC);

  // keys visible to the wave: to some row (klast_w) and to every row (kfull_w)
  const bool live = q0w < Nq;
  const int qlast_w = min(Nq - 1, q0w + QPW - 1);
  const int klast_w = CAUSAL ? min(Nk - 1, qlast_w + Nk - Nq) : Nk - 1;
  const int kfull_w = CAUSAL ? min(Nk - 1, q0w + Nk - Nq) : Nk - 1;

  const size_t qoff = (size_t)(w.b * p.Hq + hq) * Nq * D;
  const size_t kvoff = (size_t)(w.b * p.Hkv + w.hkv) * Nk * D;

  // ---- resident Q fragments (B operand of S^T = K Q^T): column = query, k = d
  bf16x8 qf[QB][DS];
  bf16x8 qlo[F32 ? QB : 1][F32 ? DS : 1];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = min(q0w + qb * 32 + (lane & 31), Nq - 1);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const size_t off = qoff + (size_t)qrow * D + ds * 16 + (lane >> 5) * 8;
      if constexpr (F32) {
        const f32x4* g = (const f32x4*)((const float*)Qp + off);
        f32x4 a = g[0], b = g[1];
        float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        split8(x, qf[qb][ds], qlo[qb][ds]);
      } else {
        qf[qb][ds] = *(const bf16x8*)((const __bf16*)Qp + off);
      }
    }
  }

  f32x16 o[QB][DB];
  float m_ref[QB], m_run[QB], lsum[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_ref[qb] = NEG_INF;
    m_run[qb] = NEG_INF;
    lsum[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb][db] = (f32x16){};
  }

  const int koff_l = k_lane_off<RS>(lane);
  const int voff_l = v_lane_off<RS>(lane);
  const __bf16* kbase = (const __bf16*)Kp + kvoff;
  const __bf16* vbase = (const __bf16*)Vp + kvoff;
  CopyPlan<D, NW> cp;
  if constexpr (!F32) {
    cp.init(wave, lane);
    if (ntiles > 0) {
      cp.issue(kbase, 0, Nk, smem, wave);
      cp.issue(vbase, 0, Nk, smem + C::TILE, wave);
    }
  }

  for (int j = 0; j < ntiles; ++j) {
    const int j0 = j * BC;
    LDS_AS const char* kt;
    LDS_AS const char* vt;
    LDS_AS const char* ktl = nullptr;
    LDS_AS const char* vtl = nullptr;
    if constexpr (F32) {
      __syncthreads();
      copy_tile_f32<D>((const float*)Kp + kvoff, j0, Nk, smem, smem + C::TILE);
      copy_tile_f32<D>((const float*)Vp + kvoff, j0, Nk, smem + 2 * C::TILE, smem + 3 * C::TILE);
      __syncthreads();
      kt = smem;
      ktl = smem + C::TILE;
      vt = smem + 2 * C::TILE;
      vtl = smem + 3 * C::TILE;
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (j + 1 < ntiles) {
        LDS_AS char* nxt = smem + ((j + 1) & 1) * 2 * C::TILE;
        cp.issue(kbase, j0 + BC, Nk, nxt, wave);
        cp.issue(vbase, j0 + BC, Nk, nxt + C::TILE, wave);
      }
      kt = smem + (j & 1) * 2 * C::TILE;
      vt = kt + C::TILE;
    }
    if (!live || j0 > klast_w) continue;  // wave-uniform: nothing visible to this wave

    // ---- S^T = K Q^T
    f32x16 s[KB][QB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = (f32x16){};
    LDS_AS const char* klane = kt + koff_l;
    LDS_AS const char* klane_lo = F32 ? ktl + koff_l : nullptr;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int off = kb * 32 * RS + ds * 32;
        const bf16x8 kf = lds_b128(klane + off);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          s[kb][qb] = mfma(kf, qf[qb][ds], s[kb][qb]);
          if constexpr (F32) s[kb][qb] = mfma(kf, qlo[qb][ds], s[kb][qb]);
        }
        if constexpr (F32) {
          const bf16x8 kl = lds_b128(klane_lo + off);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma(kl, qf[qb][ds], s[kb][qb]);
        }
      }
    }

    // ---- mask: only tiles that cross the diagonal or the end of the keys
    if (j0 + BC - 1 > kfull_w) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int query = q0w + qb * 32 + (lane & 31);
          const int kmax = (CAUSAL ? min(Nk - 1, query + Nk - Nq) : Nk - 1) - j0 - kb * 32 - (lane >> 5) * 4;
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if ((i >> 2) * 8 + (i & 3) > kmax) s[kb][qb][i] = NEG_INF;
        }
    }

    // ---- running maximum; rescale O and l only past the threshold
    bool grow = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = NEG_INF;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][qb][i]);
      mx = xhalf_max(mx);
      m_run[qb] = fmaxf(m_run[qb], mx * c);
      grow |= m_run[qb] > m_ref[qb] + TAU;
    }
    if (__ballot(grow)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float alpha = (m_run[qb] == NEG_INF) ? 1.f : __builtin_amdgcn_exp2f(m_ref[qb] - m_run[qb]);
        lsum[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[qb][db] *= alpha;
        m_ref[qb] = m_run[qb];
      }
    }

    // ---- P = 2^(S c - m_ref), row sums, bf16 operands of the second product
    bf16x8 pf[QB][PS];
    bf16x8 pl[F32 ? QB : 1][F32 ? PS : 1];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mu = (m_ref[qb] == NEG_INF) ? 0.f : m_ref[qb];
      float part = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][i], c, -mu));
          s[kb][qb][i] = pv;
          part += pv;
        }
      lsum[qb] += part;
#pragma unroll
      for (int ps = 0; ps < PS; ++ps) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = s[ps >> 1][qb][(ps & 1) * 8 + e];
        if constexpr (F32) {
          split8(x, pf[qb][ps], pl[qb][ps]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[qb][ps][e] = (__bf16)x[e];
        }
      }
    }

    // ---- O^T += V^T P^T
    LDS_AS const char* vlane = vt + voff_l;
    LDS_AS const char* vlane_lo = F32 ? vtl + voff_l : nullptr;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int ps = 0; ps < PS; ++ps) {
        const bf16x8 vf = v_frag<RS>(vlane, ps, db);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          o[qb][db] = mfma(vf, pf[qb][ps], o[qb][db]);
          if constexpr (F32) o[qb][db] = mfma(vf, pl[qb][ps], o[qb][db]);
        }
        if constexpr (F32) {
          const bf16x8 vl = v_frag<RS>(vlane_lo, ps, db);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma(vl, pf[qb][ps], o[qb][db]);
        }
      }
    }
  }

  // ---- epilogue: O / l, LSE = ln2 * (m_ref + log2 l)
  if (!live) return;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = xhalf_sum(lsum[qb]);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const int query = q0w + qb * 32 + (lane & 31);
    if (query >= Nq) continue;
    const size_t orow = qoff + (size_t)query * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = db * 32 + i4 * 8 + (lane >> 5) * 4;
        if constexpr (F32) {
          f32x4 r;
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = o[qb][db][i4 * 4 + e] * inv;
          *(f32x4*)((float*)Op + orow + d0) = r;
        } else {
          bf16x4 r;
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = (__bf16)(o[qb][db][i4 * 4 + e] * inv);
          *(bf16x4*)((__bf16*)Op + orow + d0) = r;
        }
      }
    if (LSE != nullptr && lane < 32)
      LSE[(size_t)(w.b * p.Hq + hq) * Nq + query] = lt > 0.f ? (m_ref[qb] + log2f(lt)) * LN2 : NEG_INF;
  }
}

// ---------------------------------------------------------------- launchers
// Every variant is instantiated explicitly (implicit instantiation through
// the launch expression alone does not always emit the host-side stub).
#define FA_INST(DD, CC, FF, NN)                                                                        \
  template __global__ void fa_fwd_kernel<DD, CC, FF, NN>(const void* __restrict__, const void* __restrict__, \
                                                         const void* __restrict__, void* __restrict__,    \
                                                         float* __restrict__, fa_plan_t, float);
#define FA_VARIANTS(X)                                                                                  \
  X(64, false, false, 1) X(64, false, false, 2) X(64, false, false, 4)                                  \
  X(64, true, false, 1) X(64, true, false, 2) X(64, true, false, 4)                                     \
  X(128, false, false, 1) X(128, false, false, 2) X(128, false, false, 4)                               \
  X(128, true, false, 1) X(128, true, false, 2) X(128, true, false, 4)                                  \
  X(256, false, false, 1) X(256, false, false, 2) X(256, false, false, 4)                               \
  X(256, true, false, 1) X(256, true, false, 2) X(256, true, false, 4)                                  \
  X(64, false, true, 4) X(64, true, true, 4) X(128, false, true, 4) X(128, true, true, 4)               \
  X(256, false, true, 4) X(256, true, true, 4)
FA_VARIANTS(FA_INST)

int queries_per_wave(int d, int f32) {
  if (f32) return 32;
  return d == 64 ? 64 : 32;
}

hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, const fa_plan_t& p, int d,
                      float c, int f32, hipStream_t stream) {
#define FA_CASE(DD, CC, FF, NN)                                                                      \
  if (d == DD && (p.causal != 0) == CC && (f32 != 0) == FF && p.nw == NN) {                          \
    hipLaunchKernelGGL((fa_fwd_kernel<DD, CC, FF, NN>), dim3((unsigned)p.nwg), dim3(64 * NN), 0, stream, q, k, v, \
                       o, lse, p, c);                                                                \
    return hipGetLastError();                                                                        \
  }
  FA_VARIANTS(FA_CASE)
#undef FA_CASE
  return hipErrorInvalidValue;
}

}  // namespace fa

// fa_frag.h -- MFMA operand fragments in LDS and the HBM -> LDS tile copy,
// shared by the forward and backward kernels.
//
// Operand layouts of v_mfma_f32_32x32x16_bf16 (64 lanes, h = lane / 32):
//   A (32 x 16): lane l holds row l % 32, k = 8h .. 8h + 7
//   B (16 x 32): lane l holds column l % 32, k = 8h .. 8h + 7
//   C (32 x 32): lane l holds column l % 32, rows 8 (i / 4) + 4h + i % 4 in
//                accumulator register i = 0 .. 15
// Registers 8s .. 8s + 7 of a C tile, rounded to bf16, are therefore the B
// operand of k-step s of a product that contracts over C's rows, with k
// index 8h + e standing for row 16s + 8 (e / 4) + 4h + e % 4; the A operand
// of that product must use the same row order (v_frag below).
#ifndef FA_FRAG_H
#define FA_FRAG_H

#include "fa_device.h"

namespace fa {

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
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

// Row order of tiles that are read both as row fragments and transposed.
// Within each block of 16 rows, row 4a + b of the data is stored at LDS row
// 4b + a (an involution).  With a row stride of an odd number of 16-byte
// slots, a row-fragment read (16 lanes on 16 consecutive data rows, one
// slot each) still covers 16 distinct groups of 4 banks, and a transposed
// read (32 lanes on 4 consecutive data rows, 64 bytes each) now finds its 4
// rows 4 LDS rows apart, 16 banks from each other: both are free of bank
// conflicts, which no plain row stride achieves for both.
__host__ __device__ __forceinline__ constexpr int perm16(int r) { return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3); }

// k_lane_off for a permuted tile.
template <int RS>
__device__ __forceinline__ int k_lane_off_p(int lane) { return perm16(lane & 31) * RS + (lane >> 5) * 16; }

// Transposed fragment (the layout of v_frag) from a permuted tile: data row
// ps*16 + 8j + 4h + c (h = lane / 32, c = (lane % 16) / 4) sits at LDS row
// ps*16 + 4c + 2j + h.
template <int RS>
__device__ __forceinline__ int v_lane_off_p(int lane) {
  const int g = lane >> 4, s = lane & 15;
  return (4 * (s >> 2) + (g >> 1)) * RS + (2 * (g & 1) + ((s & 3) >> 1)) * 16 + (s & 1) * 8;
}

template <int RS>
__device__ __forceinline__ bf16x8 v_frag_p(LDS_AS const char* vlane, int ps, int db) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vlane + (ps * 16) * RS + db * 64));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vlane + (ps * 16 + 2) * RS + db * 64));
  return join(a, b);
}

// HBM -> LDS copy plan of one wave: copy instruction i of the wave (global
// instruction index i*NW + wave) fills LDS bytes [ins*1024, ins*1024 + 1024)
// of the tile, lane t the slot ins*64 + t (BC*SPR is a multiple of 64, so
// the last instruction ends exactly at the end of the tile).  goff is the
// byte offset of the slot's data within the tile's rows in HBM (rows of D
// bf16, contiguous; with PERM, LDS row r takes HBM row perm16(r)); padding
// slots get an offset past any buffer range, so their load reads zero and
// writes it into the (never read) padding.
template <int D, int NW, int SPR, bool PERM = false>
struct CopyPlan {
  static constexpr int CPR = D / 8;
  static constexpr int INS = BC * SPR / 64;            // 64-lane copy instructions per tile
  static_assert(BC * SPR % 64 == 0, "whole copy instructions");
  static constexpr int MI = (INS + NW - 1) / NW;
  static constexpr unsigned OUT_OF_RANGE = 0x7ffffff0u;
  unsigned goff[MI];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int ins = i * NW + wave;
      const int sl = ins * 64 + lane;
      const int r = sl / SPR, pp = sl % SPR;
      const int src = PERM ? perm16(r) : r;  // the HBM row whose data LDS row r holds
      goff[i] = (ins < INS && pp < CPR) ? (unsigned)(src * (D * 2) + pp * 16) : OUT_OF_RANGE;
    }
  }
  // Buffer resource over a whole [Nk][D] bf16 matrix; the hardware range
  // check covers voffset + soffset, so rows >= Nk read as zero.
  __device__ __forceinline__ static __amdgpu_buffer_rsrc_t rsrc(const __bf16* base, int Nk) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, Nk * (D * 2), 0x00020000);
  }
  // Copy instruction i of this wave for the tile at byte offset soff (soff at
  // or past the range: the copy reads nothing and writes zeros).
  // Instructions past the tile (when NW does not divide INS) write into the
  // 1 KB block `spare`.
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

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

}  // namespace fa

#endif  // FA_FRAG_H

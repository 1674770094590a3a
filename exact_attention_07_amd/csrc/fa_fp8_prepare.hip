// fa_fp8_prepare.hip -- FP8 "incoherent processing" step for gfx950.
//
// "FlashAttention-3 — 闪电注意力-3", section on low precision (FP8): Q and K
// are multiplied by a random orthogonal matrix (a Hadamard matrix with random
// signs) before they are quantised, which spreads outlier channels over all
// channels while leaving Q K^T unchanged; then every tensor is quantised to
// 8-bit floating point.  Here:
//   * M = diag(signs) H_d / sqrt(d) (H_d the Sylvester Hadamard matrix),
//     applied on the right, x -> x M, to every row of Q and K; V is not
//     rotated; signs == NULL skips the rotation.  x M is computed as a fast
//     Walsh-Hadamard transform of (x * signs) scaled by 1/sqrt(d), in fp32.
//   * Q is multiplied by c0 = softmax scale * log2(e) before it is
//     quantised, so that the attention kernel's score products come out in
//     the log2 units its exponentials take;
//   * one scale per tensor: for Q and K the smallest power of two s with
//     amax|x| / s <= 448 (x = c0 * rotated Q, rotated K), so that the
//     attention kernel applies s_q s_k exactly through the matrix core's
//     power-of-two scale operands; for V s = amax|V| / 448; s = 1 for an
//     all-zero tensor; codes = e4m3(x / s), rounded to nearest even by
//     v_cvt_pk_fp8_f32 (OCP E4M3, largest finite 448).
//   * V is written transposed, [B][Hkv][d][Nkp] with Nkp = Nk rounded up to
//     a multiple of 64; within each block of 64 keys the keys are stored in
//     the order the attention kernel's P fragments use (see fa.h); padding
//     keys are zero.
//
// Work layout: a row of d elements is handled by 8 consecutive lanes, each
// holding d/8 consecutive elements; the transform runs its first log2(d/8)
// butterfly stages inside each lane and the last three across the 8 lanes
// (__shfl_xor).  Four kernels run in order on the caller's stream: zero the
// amax words; rotate + amax (a grid-stride loop, one atomicMax on the float
// bits per workgroup, all values >= 0); rotate + quantise Q and K; quantise
// and transpose V.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_kernels.h"

namespace fa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr float E4M3_MAX = 448.0f;
constexpr int FP8_BC = 64;  // key block of the V^T permutation (the attention kernel's tile)

// The permuted V^T order of a 64-key block: key k with bits
// [b5 | b4 b3 | b2 | b1 b0] goes to position [b2 | b5 | b4 b3 | b1 b0]
// (the order in which the attention kernel's P fragment holds its keys).

// Load the EPL = D/8 elements of lane `sub` (0..7) of a row as fp32.
template <int D>
__device__ __forceinline__ void load_row_part(const __bf16* row, int sub, float (&x)[D / 8]) {
  constexpr int EPL = D / 8;
#pragma unroll
  for (int c = 0; c < EPL / 8; ++c) {
    const bf16x8 v = *(const bf16x8*)(row + sub * EPL + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[c * 8 + e] = (float)v[e];
  }
}

// The signs of the lane's D/8 elements (the same for every row), loaded
// once per thread; all ones without a rotation.
template <int D>
__device__ __forceinline__ void load_signs(const float* signs, int sub, float (&sg)[D / 8]) {
  constexpr int EPL = D / 8;
  if (signs == nullptr) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) sg[e] = 1.0f;
    return;
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) sg[e] = signs[sub * EPL + e];
}

// x <- (x * signs) H_d / sqrt(d) for the row spread over 8 lanes (sg: the
// lane's signs from load_signs).
template <int D>
__device__ __forceinline__ void rotate(float (&x)[D / 8], const float (&sg)[D / 8], int sub) {
  constexpr int EPL = D / 8;
#pragma unroll
  for (int e = 0; e < EPL; ++e) x[e] *= sg[e];
  // in-lane butterflies, strides 1 .. EPL/2
#pragma unroll
  for (int h = 1; h < EPL; h <<= 1)
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      if ((e & h) == 0) {
        const float a = x[e], b = x[e + h];
        x[e] = a + b;
        x[e + h] = a - b;
      }
  // cross-lane butterflies, strides EPL, 2 EPL, 4 EPL (lanes sub ^ 1, 2, 4):
  // the partner's value by DPP (a VALU operand swizzle, no LDS round trip),
  // then x <- other + s x with s = -1 in the upper lane of the pair (the
  // fma rounds once, as the add or subtract would).  The 8 lanes of a row
  // are aligned in the wave's rows of 16: lane ^ 1 and lane ^ 2 are quad
  // permutations; lane ^ 4 is lane + 4 for banks 0 and 2 of a row (lanes
  // 0-3, 8-11: sub < 4) and lane - 4 for banks 1 and 3.
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const float o1 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x[e]), 0xB1, 0xF, 0xF, false));
    x[e] = __builtin_fmaf((sub & 1) ? -1.f : 1.f, x[e], o1);
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const float o2 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x[e]), 0x4E, 0xF, 0xF, false));
    x[e] = __builtin_fmaf((sub & 2) ? -1.f : 1.f, x[e], o2);
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int xi = __builtin_bit_cast(int, x[e]);
    int o4 = __builtin_amdgcn_update_dpp(0, xi, 0x104, 0xF, 0x5, false);   // row_shl:4, banks 0, 2
    o4 = __builtin_amdgcn_update_dpp(o4, xi, 0x114, 0xF, 0xA, false);      // row_shr:4, banks 1, 3
    x[e] = __builtin_fmaf((sub & 4) ? -1.f : 1.f, x[e], __builtin_bit_cast(float, o4));
  }
  const float inv = 1.0f / __builtin_sqrtf((float)D);
#pragma unroll
  for (int e = 0; e < EPL; ++e) x[e] *= inv;
}

// max over the workgroup (256 threads), then one atomic per workgroup; m >= 0
// so the float bit pattern orders like the value
__device__ __forceinline__ void amax_to(unsigned* word, float m) {
  __shared__ float part[4];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(word, __float_as_uint(fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]))));
}

__device__ __forceinline__ float scale_of(unsigned amax_bits) {
  const float a = __uint_as_float(amax_bits);
  return a > 0.f ? a / E4M3_MAX : 1.0f;
}

// the smallest power of two >= amax * mult / 448 (1 for an all-zero tensor)
__device__ __forceinline__ float pow2_scale_of(unsigned amax_bits, float mult) {
  const float a = __uint_as_float(amax_bits);
  if (!(a > 0.f)) return 1.0f;
  const float t = a * mult / E4M3_MAX;
  const unsigned b = __float_as_uint(t);
  if ((b & 0x007fffffu) == 0u) return t;                      // already a power of two
  return __uint_as_float(((b >> 23) + 1u) << 23);             // next power of two up
}

// 4 floats -> 4 e4m3 bytes (round to nearest even)
__device__ __forceinline__ unsigned pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (unsigned)w;
}

__global__ void zero3_kernel(unsigned* w) {
  if (threadIdx.x < 3) w[threadIdx.x] = 0u;
}

// pass 1: amax of the rotated Q and K rows (tensor 0, 1) and of V (tensor 2).
// A grid-stride loop over groups of 32 rows (the loop bound is uniform over
// the workgroup) keeps the number of workgroups, and so of atomics on the
// three words, small.
template <int D>
__global__ __launch_bounds__(256) void amax_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                   const __bf16* __restrict__ v, const float* __restrict__ signs,
                                                   long long rows_q, long long rows_k, unsigned* __restrict__ amax) {
  const int sub = threadIdx.x & 7;
  const int tensor = blockIdx.y;  // 0: Q, 1: K, 2: V
  const long long rows = tensor == 0 ? rows_q : rows_k;
  const __bf16* base = tensor == 0 ? q : tensor == 1 ? k : v;
  const bool rot = tensor < 2 && signs != nullptr;
  float sg[D / 8];
  load_signs<D>(rot ? signs : nullptr, sub, sg);
  float m = 0.f;
  for (long long r0 = (long long)blockIdx.x * 32; r0 < rows; r0 += (long long)gridDim.x * 32) {
    const long long row = r0 + (threadIdx.x >> 3);
    // rows past the end are zero (the shuffles of rotate() stay uniform)
    float x[D / 8] = {};
    if (row < rows) load_row_part<D>(base + row * D, sub, x);
    if (rot) rotate<D>(x, sg, sub);
#pragma unroll
    for (int e = 0; e < D / 8; ++e) m = fmaxf(m, fabsf(x[e]));
  }
  amax_to(&amax[tensor], m);
}

// pass 2 for Q and K: rotate again and quantise; descale written by block 0.
// A workgroup takes QK_GROUPS consecutive groups of 32 rows, so that each
// thread loads its signs once for that many rows.
constexpr int QK_GROUPS = 4;
template <int D>
__global__ __launch_bounds__(256) void quant_qk_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                       const float* __restrict__ signs, long long rows_q,
                                                       long long rows_k, uint8_t* __restrict__ q8,
                                                       uint8_t* __restrict__ k8, const unsigned* __restrict__ amax,
                                                       float* __restrict__ descale, float c0) {
  const int sub = threadIdx.x & 7;
  const int tensor = blockIdx.y;  // 0: Q, 1: K
  const long long rows = tensor == 0 ? rows_q : rows_k;
  const float mult = tensor == 0 ? c0 : 1.0f;
  const float s = pow2_scale_of(amax[tensor], mult);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    descale[tensor] = s;
    if (tensor == 0) descale[2] = scale_of(amax[2]);
  }
  const float inv = mult / s;  // s is a power of two: the division is exact
  float sg[D / 8];
  if (signs != nullptr) load_signs<D>(signs, sub, sg);
  for (int gi = 0; gi < QK_GROUPS; ++gi) {
    const long long row = ((long long)blockIdx.x * QK_GROUPS + gi) * 32 + (threadIdx.x >> 3);
    if (((long long)blockIdx.x * QK_GROUPS + gi) * 32 >= rows) break;  // uniform over the workgroup
    float x[D / 8] = {};
    const bool ok = row < rows;
    if (ok) load_row_part<D>((tensor == 0 ? q : k) + row * D, sub, x);
    if (signs != nullptr) rotate<D>(x, sg, sub);
    if (!ok) continue;
    uint8_t* out = (tensor == 0 ? q8 : k8) + row * D + sub * (D / 8);
#pragma unroll
    for (int c = 0; c < D / 8 / 16; ++c) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = c * 16 + e * 4;
        w[e] = pack4(x[i] * inv, x[i + 1] * inv, x[i + 2] * inv, x[i + 3] * inv);
      }
      *(u32x4*)(out + c * 16) = w;
    }
    if constexpr (D / 8 < 16) {  // d = 64: 8 bytes per lane
      unsigned w0 = pack4(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv);
      unsigned w1 = pack4(x[4] * inv, x[5] * inv, x[6] * inv, x[7] * inv);
      *(unsigned long long*)out = ((unsigned long long)w1 << 32) | w0;
    }
  }
}

// pass 2 for V: quantise a block of 64 keys x D of one (b, h_kv), write it
// transposed with the keys of the block permuted; keys >= Nk are zero.
template <int D>
__global__ __launch_bounds__(256) void quant_v_kernel(const __bf16* __restrict__ v, int Nk, int Nkp,
                                                      uint8_t* __restrict__ v8t, const unsigned* __restrict__ amax) {
  __shared__ uint8_t tile[FP8_BC][D + 4];
  const int nblk = Nkp / FP8_BC;
  const int blk = (int)(blockIdx.x % nblk);          // key block
  const long long head = blockIdx.x / nblk;          // b * Hkv + h_kv
  const float inv = 1.0f / scale_of(amax[2]);
  const __bf16* src = v + head * (long long)Nk * D;
  // load + quantise: 64 rows x D, 8 elements per thread-step
  for (int idx = threadIdx.x; idx < FP8_BC * D / 8; idx += blockDim.x) {
    const int r = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
    const int key = blk * FP8_BC + r;
    float x[8] = {};
    if (key < Nk) {
      const bf16x8 t = *(const bf16x8*)(src + (long long)key * D + c8);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (float)t[e] * inv;
    }
    const unsigned w0 = pack4(x[0], x[1], x[2], x[3]), w1 = pack4(x[4], x[5], x[6], x[7]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[r][c8 + e] = (uint8_t)(w0 >> (8 * e));
      tile[r][c8 + 4 + e] = (uint8_t)(w1 >> (8 * e));
    }
  }
  __syncthreads();
  // write: row d of V^T gets 64 bytes, byte p = the key that the permuted
  // order puts at position p
  uint8_t* dst = v8t + head * (long long)D * Nkp + (long long)blk * FP8_BC;
  for (int idx = threadIdx.x; idx < D * (FP8_BC / 4); idx += blockDim.x) {
    const int d = idx / (FP8_BC / 4), p4 = (idx % (FP8_BC / 4)) * 4;
    unsigned w = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // inverse permutation: the key stored at position p
      const int p = p4 + e;
      const int key = (((p >> 5) & 1) << 2) | (((p >> 4) & 1) << 5) | (((p >> 2) & 3) << 3) | (p & 3);
      w |= (unsigned)tile[key][d] << (8 * e);
    }
    *(unsigned*)(dst + (long long)d * Nkp + p4) = w;
  }
}

}  // namespace

template <int D>
static hipError_t launch_prepare_d(const void* q, const void* k, const void* v, void* q8, void* k8, void* v8t,
                                   float* descale, unsigned* amax, const float* signs, float c0, long long rows_q,
                                   long long rows_k, long long heads_kv, int Nk, hipStream_t stream) {
  const int Nkp = (Nk + FP8_BC - 1) / FP8_BC * FP8_BC;
  hipLaunchKernelGGL(zero3_kernel, dim3(1), dim3(64), 0, stream, amax);
  const long long rmax = rows_q > rows_k ? rows_q : rows_k;
  // at most 512 workgroups per tensor (two per CU): each ends with one
  // same-address atomic, which serialise; measured on the fp8 workload,
  // 1024 workgroups 3.5 % slower, 256 slower again with the rotation (too
  // few rows rotating at once)
  const long long groups = (rmax + 31) / 32;
  const dim3 g1((unsigned)(groups < 512 ? groups : 512), 3);
  hipLaunchKernelGGL(amax_kernel<D>, g1, dim3(256), 0, stream, (const __bf16*)q, (const __bf16*)k,
                     (const __bf16*)v, signs, rows_q, rows_k, amax);
  const dim3 g2((unsigned)((groups + QK_GROUPS - 1) / QK_GROUPS), 2);
  hipLaunchKernelGGL(quant_qk_kernel<D>, g2, dim3(256), 0, stream, (const __bf16*)q, (const __bf16*)k, signs, rows_q,
                     rows_k, (uint8_t*)q8, (uint8_t*)k8, (const unsigned*)amax, descale, c0);
  const dim3 g3((unsigned)((long long)(Nkp / FP8_BC) * heads_kv));
  hipLaunchKernelGGL(quant_v_kernel<D>, g3, dim3(256), 0, stream, (const __bf16*)v, Nk, Nkp, (uint8_t*)v8t,
                     (const unsigned*)amax);
  return hipGetLastError();
}

bool fp8_prepare_too_large(int B, int Hq, int Hkv, int Nq, int Nk) {
  // every grid is one-dimensional with fewer than 2^31 workgroups
  const long long rows_q = (long long)B * Hq * Nq, rows_k = (long long)B * Hkv * Nk;
  const long long rmax = rows_q > rows_k ? rows_q : rows_k;
  return (rmax + 31) / 32 > 0x7fffffffLL ||
         (long long)((Nk + FP8_BC - 1) / FP8_BC) * ((long long)B * Hkv) > 0x7fffffffLL;
}

hipError_t launch_fp8_prepare(const void* q, const void* k, const void* v, void* q8, void* k8, void* v8t,
                              float* descale, unsigned* amax, const float* signs, float c0, int B, int Hq, int Hkv,
                              int Nq, int Nk, int d, hipStream_t stream) {
  const long long rows_q = (long long)B * Hq * Nq, rows_k = (long long)B * Hkv * Nk;
  const long long heads_kv = (long long)B * Hkv;
  if (fp8_prepare_too_large(B, Hq, Hkv, Nq, Nk)) return hipErrorInvalidValue;
  if (d == 64) return launch_prepare_d<64>(q, k, v, q8, k8, v8t, descale, amax, signs, c0, rows_q, rows_k,
                                                   heads_kv, Nk, stream);
  if (d == 128) return launch_prepare_d<128>(q, k, v, q8, k8, v8t, descale, amax, signs, c0, rows_q, rows_k,
                                                   heads_kv, Nk, stream);
  if (d == 256) return launch_prepare_d<256>(q, k, v, q8, k8, v8t, descale, amax, signs, c0, rows_q, rows_k,
                                                   heads_kv, Nk, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa

// fa_issue.hip -- the cost of vector work beside the matrix core: loops of
// the MFMAs the attention kernels use (bf16 32x32x16; e4m3 32x32x64, plain,
// with E8M0 scale operands, or the two alternating as in the fp8 kernel)
// with exponentials, e4m3 packings and FMAs beside them, two waves per SIMD
// (the grid of the MFMA ceiling loop).  Timed against the MFMA-only loop of
// the same instruction, they price the per-score vector work of the
// attention kernels in matrix-pipe time, and show whether moving
// exponentials onto the FMA units (a polynomial for exp2) can pay.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_kernels.h"

namespace fa {
namespace {

typedef __bf16 bf16x8i __attribute__((ext_vector_type(8)));
typedef float f32x16i __attribute__((ext_vector_type(16)));
typedef int i32x8i __attribute__((ext_vector_type(8)));

// Matrix instruction of a case: bf16 32x32x16; e4m3 32x32x64 plain; the
// same with E8M0 scale operands (2^0 on both); the two e4m3 forms
// alternating, as the fp8 kernel's S and P V products do.
enum IssueMfma { MFMA_BF16 = 0, MFMA_FP8 = 1, MFMA_FP8_SCALED = 2, MFMA_FP8_ALTERNATING = 3 };

__device__ __forceinline__ unsigned mix(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Each wave runs `iters` rounds; a round is NM MFMAs of kind KIND (random
// operands, as in the ceiling loop) with NE exponentials (v_exp_f32), NC
// e4m3 packings (v_cvt_pk_fp8_f32) and NF fused multiply-adds spread evenly
// over them, each kind on 8 independent chains.  Timed against the
// MFMA-only round of the same instruction, the rounds show what a mix of
// vector work costs the matrix pipe, and whether replacing an exponential by
// a polynomial on the FMA units (one v_exp_f32 by seven fast instructions)
// can pay.
template <int NM, int NE, int NC, int NF, int KIND>
__global__ __launch_bounds__(256) void issue_loop_kernel(float* __restrict__ out, int iters, int e8m0_one) {
  const unsigned tid = blockIdx.x * blockDim.x + threadIdx.x;
  f32x16i acc[4] = {};
  bf16x8i a[2], b[2];
  i32x8i a8[2], b8[2];
  for (int s = 0; s < 2; ++s)
    for (int i = 0; i < 8; ++i) {
      const unsigned h = mix(tid * 131u + s * 17u + i * 7u);
      a[s][i] = (__bf16)((float)(h & 0xffff) / 16384.0f - 2.0f);
      b[s][i] = (__bf16)((float)(h >> 16) / 16384.0f - 2.0f);
      // e4m3 bytes with exponent fields below 15 (no NaN codes)
      a8[s][i] = (int)((h & 0x77777777u) | 0x08080808u);
      b8[s][i] = (int)(mix(h) & 0xf7f7f7f7u & ~0x80808080u);
    }
  float e[8], f[8], x[8];
  int c[8];
  for (int i = 0; i < 8; ++i) {
    e[i] = -(float)(tid & 7) - 0.125f * i;
    f[i] = 0.5f + 0.01f * i;
    x[i] = (float)(tid & 3) + 0.5f * i;
    c[i] = (int)tid;
  }
  const float g = 0.999f, h = 0.001f;
  constexpr int SLOTS = NM > 0 ? NM : 1;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < SLOTS; ++m) {
      if constexpr (NM > 0) {
        if constexpr (KIND == MFMA_BF16) {
          acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m & 1], b[(m >> 1) & 1], acc[m & 3], 0, 0, 0);
        } else if (KIND == MFMA_FP8 || (KIND == MFMA_FP8_ALTERNATING && (m & 1) == 1)) {
          acc[m & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8[m & 1], b8[(m >> 1) & 1], acc[m & 3], 0, 0, 0,
                                                                        0, 0, 0);
        } else {
          acc[m & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8[m & 1], b8[(m >> 1) & 1], acc[m & 3], 0, 0, 0,
                                                                        e8m0_one, 0, e8m0_one);
        }
      }
#pragma unroll
      for (int k = m * NE / SLOTS; k < (m + 1) * NE / SLOTS; ++k) e[k % 8] = __builtin_amdgcn_exp2f(e[k % 8]);
#pragma unroll
      for (int k = m * NC / SLOTS; k < (m + 1) * NC / SLOTS; ++k)
        c[k % 8] = __builtin_amdgcn_cvt_pk_fp8_f32(x[k % 8], x[(k + 1) % 8], c[k % 8], false);
#pragma unroll
      for (int k = m * NF / SLOTS; k < (m + 1) * NF / SLOTS; ++k) f[k % 8] = __builtin_fmaf(f[k % 8], g, h);
    }
  }
  float s = 0.f;
  for (int i = 0; i < 8; ++i) s += e[i] + f[i] + (float)c[i];
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 16; ++j) s += acc[i][j];
  out[tid] = s;
}

}  // namespace

// The rounds of the issue-cost loop: {MFMAs, exponentials, e4m3 packings,
// FMAs, MFMA kind}.  Four bf16 MFMAs (or two e4m3 ones, each covering four
// times the contraction in twice the cycles) take as long as the bf16
// kernel spends on one score per lane for each of 4 MFMAs' worth of keys;
// per four bf16 MFMAs that kernel issues 4 exponentials and ~10 fast
// instructions (4 FMAs, 4 adds, 2 bf16 packings), the fp8 kernel per two
// e4m3 MFMAs 8 exponentials, 4 e4m3 packings and ~8 adds, about 9, 4 and 16
// as its counters see them (slow path included).
static const int kIssueCases[][5] = {
    {4, 0, 0, 0, MFMA_BF16},   // matrix work alone
    {0, 8, 0, 0, MFMA_BF16},   // exponentials alone
    {0, 0, 0, 16, MFMA_BF16},  // FMAs alone
    {0, 8, 0, 16, MFMA_BF16},  // both, no matrix work
    {4, 8, 0, 0, MFMA_BF16},   {4, 16, 0, 0, MFMA_BF16},  {4, 0, 0, 16, MFMA_BF16}, {4, 0, 0, 32, MFMA_BF16},
    {4, 4, 0, 10, MFMA_BF16},  // the bf16 kernel's mix
    {4, 3, 0, 17, MFMA_BF16},  // ... with a quarter of its exponentials on the FMA units
    {4, 2, 0, 24, MFMA_BF16},  // ... with half
    {4, 8, 4, 8, MFMA_BF16},   // the fp8 kernel's mix beside bf16 MFMAs
    {4, 6, 4, 22, MFMA_BF16},  // ... with a quarter of its exponentials on the FMA units
    {4, 4, 4, 36, MFMA_BF16},  // ... with half
    {2, 0, 0, 0, MFMA_FP8},    // e4m3 matrix work alone
    {2, 8, 4, 8, MFMA_FP8},    // the fp8 kernel's mix beside its own MFMAs
    {2, 0, 0, 0, MFMA_FP8_SCALED},
    {2, 8, 4, 8, MFMA_FP8_SCALED},
    {2, 0, 0, 0, MFMA_FP8_ALTERNATING},
    {2, 8, 4, 8, MFMA_FP8_ALTERNATING},
    {2, 9, 4, 16, MFMA_FP8_ALTERNATING},  // the fp8 kernel's counted mix
};
constexpr int kNumIssueCases = sizeof(kIssueCases) / sizeof(kIssueCases[0]);

int issue_cost_cases() { return kNumIssueCases; }

bool issue_cost_case(int i, int* mfmas, int* exps, int* cvts, int* fmas) {
  if (i < 0 || i >= kNumIssueCases) return false;
  *mfmas = kIssueCases[i][0];
  *exps = kIssueCases[i][1];
  *cvts = kIssueCases[i][2];
  *fmas = kIssueCases[i][3];
  return true;
}

bool issue_cost_case_mfma(int i, int* kind) {
  if (i < 0 || i >= kNumIssueCases) return false;
  *kind = kIssueCases[i][4];
  return true;
}

hipError_t launch_issue_cost(float* out, int i, int iters, hipStream_t stream) {
  if (iters < 1 || i < 0 || i >= kNumIssueCases) return hipErrorInvalidValue;
  const unsigned nwg = mfma_ceiling_workgroups();
#define FA_ISSUE_CASE(NM, NE, NC, NF, KK)                                                                    \
  if (kIssueCases[i][0] == NM && kIssueCases[i][1] == NE && kIssueCases[i][2] == NC && kIssueCases[i][3] == NF && \
      kIssueCases[i][4] == KK) {                                                                              \
    hipLaunchKernelGGL((issue_loop_kernel<NM, NE, NC, NF, KK>), dim3(nwg), dim3(256), 0, stream, out, iters, 127); \
    return hipGetLastError();                                                                                \
  }
  FA_ISSUE_CASE(4, 0, 0, 0, 0) FA_ISSUE_CASE(0, 8, 0, 0, 0) FA_ISSUE_CASE(0, 0, 0, 16, 0) FA_ISSUE_CASE(0, 8, 0, 16, 0)
  FA_ISSUE_CASE(4, 8, 0, 0, 0) FA_ISSUE_CASE(4, 16, 0, 0, 0) FA_ISSUE_CASE(4, 0, 0, 16, 0) FA_ISSUE_CASE(4, 0, 0, 32, 0)
  FA_ISSUE_CASE(4, 4, 0, 10, 0) FA_ISSUE_CASE(4, 3, 0, 17, 0) FA_ISSUE_CASE(4, 2, 0, 24, 0)
  FA_ISSUE_CASE(4, 8, 4, 8, 0) FA_ISSUE_CASE(4, 6, 4, 22, 0) FA_ISSUE_CASE(4, 4, 4, 36, 0)
  FA_ISSUE_CASE(2, 0, 0, 0, 1) FA_ISSUE_CASE(2, 8, 4, 8, 1) FA_ISSUE_CASE(2, 0, 0, 0, 2) FA_ISSUE_CASE(2, 8, 4, 8, 2)
  FA_ISSUE_CASE(2, 0, 0, 0, 3) FA_ISSUE_CASE(2, 8, 4, 8, 3) FA_ISSUE_CASE(2, 9, 4, 16, 3)
#undef FA_ISSUE_CASE
  return hipErrorInvalidValue;
}

}  // namespace fa

// fa_ceiling.hip -- the measured MFMA ceiling: a loop of nothing but dense
// matrix instructions, the same shapes the attention kernels use
// (v_mfma_f32_32x32x16_bf16, v_mfma_f32_32x32x64_f8f6f4), two waves per
// SIMD, operands that change from instruction to instruction.
//
// The attention path is a dense contraction, so its roofline is the MFMA
// rate; on a power-capped chip the clock under a sustained matrix load, and
// therefore the reachable rate, depends on how much the operand bits toggle.
// Timed beside the attention kernel, this loop gives the rate the chip
// sustains for pure matrix work on random data at the same moment, the
// second denominator the measurement reports next to the nominal peak.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_kernels.h"

namespace fa {
namespace {

typedef __bf16 bf16x8c __attribute__((ext_vector_type(8)));
typedef float f32x16c __attribute__((ext_vector_type(16)));
typedef int i32x8c __attribute__((ext_vector_type(8)));

__device__ __forceinline__ unsigned mix(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Each wave: `iters` rounds of 16 independent MFMAs over 4 accumulators,
// operand sets rotating among 4 (A changes every instruction, B every 4).
// random = 0: every operand element is a constant (the low-toggle case).
// One float per lane is stored so that nothing is optimised away.
template <bool FP8>
__global__ __launch_bounds__(256) void mfma_loop_kernel(float* __restrict__ out, int iters, int random) {
  const unsigned tid = blockIdx.x * blockDim.x + threadIdx.x;
  f32x16c acc[4] = {};
  if constexpr (!FP8) {
    bf16x8c a[4], b[4];
    for (int s = 0; s < 4; ++s)
      for (int i = 0; i < 8; ++i) {
        const unsigned h = mix(tid * 131u + s * 17u + i * 7u);
        a[s][i] = (__bf16)(random ? (float)(h & 0xffff) / 16384.0f - 2.0f : 0.5f);
        b[s][i] = (__bf16)(random ? (float)(h >> 16) / 16384.0f - 2.0f : 0.25f);
      }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int m = 0; m < 16; ++m)
        acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m & 3], b[(m >> 2) & 3], acc[m & 3], 0, 0, 0);
    }
  } else {
    i32x8c a[4], b[4];
    for (int s = 0; s < 4; ++s)
      for (int i = 0; i < 8; ++i) {
        const unsigned h = mix(tid * 131u + s * 17u + i * 7u);
        // e4m3 bytes with exponent fields below 15 (no NaN codes); constant:
        // 0x38 = 1.0 in every byte
        const unsigned r = (h & 0x77777777u) | 0x08080808u;
        a[s][i] = (int)(random ? r : 0x38383838u);
        b[s][i] = (int)(random ? mix(h) & 0xf7f7f7f7u & ~0x80808080u : 0x38383838u);
      }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int m = 0; m < 16; ++m)
        acc[m & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[m & 3], b[(m >> 2) & 3], acc[m & 3], 0, 0,
                                                                      0, 0, 0, 0);
    }
  }
  float s = 0.f;
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 16; ++j) s += acc[i][j];
  out[tid] = s;
}

}  // namespace

// Two workgroups of four waves per CU: two waves per SIMD.
unsigned mfma_ceiling_workgroups() {
  const int cus = cu_count();
  return 2u * (unsigned)(cus > 0 ? cus : 256);
}

double mfma_ceiling_flops(int fp8, int iters) {
  const double per_ins = fp8 ? 2.0 * 32 * 32 * 64 : 2.0 * 32 * 32 * 16;
  return (double)mfma_ceiling_workgroups() * 4.0 * 16.0 * iters * per_ins;
}

hipError_t launch_mfma_ceiling(float* out, int fp8, int iters, int random, hipStream_t stream) {
  if (iters < 1) return hipErrorInvalidValue;
  const unsigned nwg = mfma_ceiling_workgroups();
  if (fp8)
    hipLaunchKernelGGL(mfma_loop_kernel<true>, dim3(nwg), dim3(256), 0, stream, out, iters, random);
  else
    hipLaunchKernelGGL(mfma_loop_kernel<false>, dim3(nwg), dim3(256), 0, stream, out, iters, random);
  return hipGetLastError();
}

}  // namespace fa

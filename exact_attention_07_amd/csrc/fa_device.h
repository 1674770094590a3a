// fa_device.h -- device-side definitions shared by the attention kernels.
#ifndef FA_DEVICE_H
#define FA_DEVICE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

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
constexpr float TAU_EXP2 = 256.0f;  // 2^TAU

// s_waitcnt vmcnt(N): wait until at most N vector memory operations of this
// wave are outstanding (they complete in issue order for loads into LDS)
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
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

}  // namespace fa

#endif  // FA_DEVICE_H

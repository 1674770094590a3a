// fa_kernels.h -- internal interface between the C-ABI layer and the kernels.
#ifndef FA_KERNELS_H
#define FA_KERNELS_H

#include <hip/hip_runtime.h>

#include "plan.h"

namespace fa {

// Query rows per wave of the forward kernel for head dimension d.
int queries_per_wave(int d, int f32);

// Enqueue the forward kernel.  c = scale * log2(e).  f32 selects fp32
// operands (split into bf16 hi/lo parts inside the kernel).
hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, const fa_plan_t& p, int d,
                      float c, int f32, hipStream_t stream);

}  // namespace fa

#endif

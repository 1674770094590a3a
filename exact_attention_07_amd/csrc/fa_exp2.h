// fa_exp2.h -- 2^x on the FMA pipe, for the part of the exponentials that
// fa_fwd_exp2_emulated takes off the hardware exponential unit
// ("FlashAttention-4震撼发布：性能再攀新高", second algorithmic improvement:
// some exponentials are computed by a polynomial on the FMA units).
//
// x = n + f with n = floor(x) and f in [0, 1); 2^f ~ p(f), the cubic of
// fa_exp2_coef.h (minimax in the relative error over [0, 1], largest
// relative error 7.5e-5, fitted by exp2_fit.py); 2^x = p(f) * 2^n by
// v_ldexp_f32.  Inputs below -200 (a masked score is -inf) are raised to
// -200, whose result underflows to exactly 0, so masked keys still weigh
// nothing.  Eight VALU instructions (max, floor, subtract, three FMAs, the
// conversion of n, ldexp) against one v_exp_f32.
#pragma once
#include <hip/hip_runtime.h>

#include "fa_exp2_coef.h"

namespace fa {

__device__ __forceinline__ float exp2_poly(float x) {
  x = __builtin_fmaxf(x, -200.0f);
  const float n = __builtin_floorf(x);
  const float f = x - n;
  float p = FA_EXP2_C3;
  p = __builtin_fmaf(p, f, FA_EXP2_C2);
  p = __builtin_fmaf(p, f, FA_EXP2_C1);
  p = __builtin_fmaf(p, f, FA_EXP2_C0);
  return __builtin_ldexpf(p, (int)n);
}

}  // namespace fa

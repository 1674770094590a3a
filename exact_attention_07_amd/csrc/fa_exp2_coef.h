// fa_exp2_coef.h -- coefficients of p(f) ~ 2^f on [0, 1), lowest first,
// minimax in the relative error (Remez exchange, degree 3), rounded to
// fp32; levelled relative error of the exact-coefficient fit 7.478e-05.
// Written by exact_attention_07_amd/exp2_fit.py; do not edit.
#pragma once
#define FA_EXP2_C0 0x1.fff6320000000p-1f  /* 0.9999251961708069 */
#define FA_EXP2_C1 0x1.64444c0000000p-1f  /* 0.6958335638046265 */
#define FA_EXP2_C2 0x1.cefc4c0000000p-3f  /* 0.22606715559959412 */
#define FA_EXP2_C3 0x1.3f96a40000000p-4f  /* 0.07802452147006989 */

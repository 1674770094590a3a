// fa_api.cpp -- the extern "C" entry points of libfa.so (declared in fa.h):
// argument validation on the host, launch planning, dispatch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "fa.h"
#include "fa_kernels.h"
#include "plan.h"

namespace {

constexpr double LOG2E = 1.4426950408889634074;
// Enough workgroups to give every one of the 256 CUs several in turn.
constexpr long long MIN_WORKGROUPS = 1024;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by the forward entry points; nothing touches HIP.
fa_status validate(const void* q, const void* k, const void* v, const void* o, const void* lse, int B, int Hq,
                   int Hkv, int Nq, int Nk, int d, float scale, int causal) {
  if (!q || !k || !v || !o) return FA_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128 && d != 256) return FA_ERR_HEAD_DIM;
  if (Hq % Hkv != 0) return FA_ERR_GQA_RATIO;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
    return FA_ERR_ALIGN;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
  if (causal != 0 && causal != 1) return FA_ERR_FLAG;
  // every element offset must fit in 63 bits, and one key/value head (the
  // range of a buffer resource) in 31 bits
  const double elems = (double)B * (double)(Hq > Hkv ? Hq : Hkv) * (double)(Nq > Nk ? Nq : Nk) * d;
  if (elems > 9.0e18) return FA_ERR_SHAPE;
  if ((double)Nk * d * 4.0 >= 2147483648.0) return FA_ERR_SHAPE;
  return FA_OK;
}

fa_status forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Nq,
                  int Nk, int d, float scale, int causal, void* stream, int f32) {
  fa_status st = validate(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal);
  if (st != FA_OK) return st;
  const int qpw = fa::queries_per_wave(d, f32);
  // the fp32 path is instantiated for 4-wave workgroups only
  // bf16: up to 4 waves per workgroup (two workgroups share a CU at d <= 128)
  const fa_plan_t p = f32 ? fa_make_plan(B, Hq, Hkv, Nq, Nk, causal, qpw, 4)
                          : fa_choose_plan(B, Hq, Hkv, Nq, Nk, causal, qpw, MIN_WORKGROUPS, 4);
  if (p.nwg > 0x7fffffffLL) return FA_ERR_SHAPE;
  const float c = (float)((double)scale * LOG2E);
  hipError_t e = fa::launch_fwd(q, k, v, o, lse, p, d, c, f32, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

int fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid or too large shape (B, Hq, Hkv, Nq, Nk)";
    case FA_ERR_HEAD_DIM: return "head dimension must be 64, 128 or 256";
    case FA_ERR_GQA_RATIO: return "Hq must be a multiple of Hkv";
    case FA_ERR_ALIGN: return "pointers must be 16-byte aligned";
    case FA_ERR_SCALE: return "scale must be finite and > 0";
    case FA_ERR_HIP: return "HIP launch failed";
    case FA_ERR_FLAG: return "causal must be 0 or 1";
  }
  return "unknown status";
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Nq,
                 int Nk, int d, float scale, int causal, void* stream) {
  return forward(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, stream, 0);
}

fa_status fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int Hq, int Hkv,
                     int Nq, int Nk, int d, float scale, int causal, void* stream) {
  return forward(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, stream, 1);
}

}  // extern "C"

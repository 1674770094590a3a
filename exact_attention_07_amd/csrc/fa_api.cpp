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
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Shape checks shared by every entry point.
fa_status validate_shape(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128 && d != 256) return FA_ERR_HEAD_DIM;
  if (Hq % Hkv != 0) return FA_ERR_GQA_RATIO;
  const double elems = (double)B * (double)(Hq > Hkv ? Hq : Hkv) * (double)(Nq > Nk ? Nq : Nk) * d;
  if (elems > 9.0e18) return FA_ERR_SHAPE;
  // one key/value head (the range of a buffer resource) fits in 31 bits
  if (((double)Nk + 64.0) * d * 4.0 >= 2147483648.0) return FA_ERR_SHAPE;
  return FA_OK;
}

// Checks shared by the forward entry points; nothing touches HIP.
fa_status validate(const void* q, const void* k, const void* v, const void* o, const void* lse, int B, int Hq,
                   int Hkv, int Nq, int Nk, int d, float scale, int causal) {
  if (!q || !k || !v || !o) return FA_ERR_NULL;
  const fa_status st = validate_shape(B, Hq, Hkv, Nq, Nk, d);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
    return FA_ERR_ALIGN;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
  if (causal != 0 && causal != 1) return FA_ERR_FLAG;
  return FA_OK;
}

enum { KIND_BF16 = 0, KIND_F32 = 1, KIND_FP8 = 2 };
fa_plan_t plan_for(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, int kind);

fa_status forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Nq,
                  int Nk, int d, float scale, int causal, void* stream, int f32, int emu = 0) {
  fa_status st = validate(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal);
  if (st != FA_OK) return st;
  const fa_plan_t p = plan_for(B, Hq, Hkv, Nq, Nk, d, causal, f32 ? KIND_F32 : KIND_BF16);
  if (p.nwg > 0x7fffffffLL) return FA_ERR_SHAPE;
  const float c = (float)((double)scale * LOG2E);
  hipError_t e = fa::launch_fwd(q, k, v, o, lse, p, d, c, f32, nullptr, nullptr, (hipStream_t)stream, emu);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// bf16 with few query rows: the G query heads of a GQA group share the 32
// query columns of one wave, or of a few (plan.h, fa_make_packed_plan).
bool packable(int Hq, int Hkv, int Nq, int d) {
  return Hq / Hkv > 1 && Nq <= 16 && fa_packed_waves(Hq / Hkv, Nq) <= (d == 128 ? 8 : 4);
}

fa_plan_t plan_for(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, int kind) {
  if (kind == KIND_BF16 && packable(Hq, Hkv, Nq, d)) return fa_make_packed_plan(B, Hq, Hkv, Nq, Nk, causal);
  const int qpw = fa::queries_per_wave(d, kind == KIND_F32);
  if (kind == KIND_F32) return fa_make_plan(B, Hq, Hkv, Nq, Nk, causal, qpw, 4);
  return fa_forward_plan(B, Hq, Hkv, Nq, Nk, causal, d, kind == KIND_FP8, qpw);
}

// Key-split plan of the bf16 path.  Few query rows: one workgroup holds all
// query heads of a GQA group, packed into the query columns of its waves
// when Nq <= 16, else one head per wave (up to the wave limit), so each K/V
// tile is read once for all of them.  Then the keys are split into ranges
// until the grid has MIN_WORKGROUPS workgroups (nsplit_req = 0), or into
// nsplit_req ranges of equal tile counts (the last may be shorter; fewer
// ranges result when nsplit_req does not divide the tiles evenly).
fa_plan_t plan_splitkv(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, int nsplit_req) {
  const int qpw = fa::queries_per_wave(d, 0);
  fa_plan_t base;
  if (packable(Hq, Hkv, Nq, d)) {
    base = fa_make_packed_plan(B, Hq, Hkv, Nq, Nk, causal);
  } else if (Nq <= qpw) {
    const int max_nw = d == 128 ? 8 : 4;
    int nw = 1;
    while (nw * 2 <= max_nw && (Hq / Hkv) % (nw * 2) == 0) nw *= 2;
    base = fa_make_plan(B, Hq, Hkv, Nq, Nk, causal, qpw, nw);
  } else {
    base = plan_for(B, Hq, Hkv, Nq, Nk, d, causal, KIND_BF16);
  }
  const long long tiles = ((long long)Nk + 63) / 64;
  long long want = nsplit_req;
  // packed plans: two workgroups per CU (LDS), so 512 fill the chip once;
  // more only queue behind them (measured on decoding, B8 Hq32 Hkv8 Nk32K
  // d128: 8 ranges 0.197 ms, 16 ranges 0.214 ms)
  const long long target = base.pack > 1 ? 512 : MIN_WORKGROUPS;
  if (want == 0) want = base.nwg >= target ? 1 : (target + base.nwg - 1) / base.nwg;
  if (want > tiles) want = tiles;
  if (want <= 1) return base;
  const int tps = (int)((tiles + want - 1) / want);
  return fa_split_plan(base, tps, 64);
}

size_t splitkv_workspace_bytes(const fa_plan_t& p, int d) {
  if (p.nsplit <= 1) return 0;
  const size_t rows = (size_t)p.B * p.Hq * p.Nq;
  return (size_t)p.nsplit * rows * (size_t)(d + 1) * sizeof(float);
}

// Backward plans.  dQ: the forward kernel's plan (32 query rows per wave).
// dK/dV: key blocks of up to bwd_dkdv_max_waves waves (a workgroup of that
// size fills a CU on its own), and enough workgroups through fewer waves or
// split head groups (plan_bwd_dkdv).
constexpr long long MIN_KV_WORKGROUPS = 512;

// The dQ kernel has the forward kernel's shape, K/V ring and occupancy, and
// the forward's wave-count rule (plan.h, fa_forward_plan) measured the
// fastest or within 4 % of it over 13 shapes (d = 64, 128, 256), up to 3.6x
// faster than the most waves that still leave 1024 workgroups.
fa_plan_t plan_bwd_dq(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal) {
  return fa_forward_plan(B, Hq, Hkv, Nq, Nk, causal, d, 0, 32);
}

fa_kvplan_t plan_bwd_dkdv(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal) {
  const int kpw = fa::bwd_keys_per_wave(d);
  const int G = Hq / Hkv, max_nw = fa::bwd_dkdv_max_waves(d);
  // the fewest head parts (a divisor of G) that give at least `target`
  // workgroups: each part adds its heads' share of dK and dV into an fp32
  // partial sum in the workspace
  auto split_to = [&](const fa_kvplan_t& p, long long target) {
    if (p.nwg >= target || G == 1) return p;
    for (int parts = 2; parts < G; ++parts)
      if (G % parts == 0 && p.nwg * parts >= target) return fa_split_kvplan_heads(p, parts);
    return fa_split_kvplan_heads(p, G);
  };
  const fa_kvplan_t big = fa_make_kvplan(B, Hq, Hkv, Nq, Nk, causal, kpw, max_nw);
  // d = 256: one workgroup fills a CU's LDS whatever its wave count.  With
  // G > 1 the most waves, heads split up to 256 workgroups, 512 if causal
  // (B2 H16 Hkv1 N4096 causal: 4377 us at one wave per workgroup, 746 us with
  // 4 waves and 8 parts); with G = 1 fewer waves while under 256 workgroups
  // (B1 H8 N2048: 2 waves 3 % faster than 4).
  if (d == 256) {
    if (G > 1) return split_to(big, causal ? 512 : 256);
    for (int nw = max_nw; nw > 1; nw >>= 1) {
      const fa_kvplan_t p = fa_make_kvplan(B, Hq, Hkv, Nq, Nk, causal, kpw, nw);
      if (p.nwg >= 256) return p;
    }
    return fa_make_kvplan(B, Hq, Hkv, Nq, Nk, causal, kpw, 1);
  }
  // d = 64 with G > 1.  Causal with Nq >= Nk / 2, where the key blocks'
  // work differs most: 2-wave workgroups, heads split up to 2048 workgroups
  // (B2 H32 Hkv8 N4096: 404 us against 546 us at 4 waves unsplit).
  // Otherwise every key block sees about the same rows: 4 waves, heads split
  // only up to 256 workgroups (B2 H32 Hkv8 Nq1024 Nk8192 causal: unsplit
  // 299 us, 2 parts 337 us).
  if (d == 64 && G > 1) {
    if (causal && 2LL * Nq >= Nk) return split_to(fa_make_kvplan(B, Hq, Hkv, Nq, Nk, causal, kpw, 2), 2048);
    return split_to(big, 256);
  }
  // d = 128 with G > 1: 8 waves (256 such workgroups already hold 8 waves
  // on every CU), heads split up to 256 workgroups, 512 if causal (B1 H32
  // Hkv4 N16384 causal: 4 waves 6836 us, 8 waves and 2 parts 3998 us; B2 H32
  // Hkv8 N4096: 4 waves 1141 us, 8 waves 948 us)
  if (d == 128 && G > 1) return split_to(big, causal ? 512 : 256);
  // d = 128 with G = 1, and d = 64 with G = 1: fewer waves while under 512
  // workgroups, but at d = 128 never fewer than 2 (one-wave workgroups leave
  // most of a CU idle: B1 H8 N2048: 132 us against 69 us with two)
  const int min_nw = d == 128 ? 2 : 1;
  for (int nw = max_nw; nw > min_nw; nw >>= 1) {
    const fa_kvplan_t p = fa_make_kvplan(B, Hq, Hkv, Nq, Nk, causal, kpw, nw);
    if (p.nwg >= MIN_KV_WORKGROUPS) return p;
  }
  return fa_make_kvplan(B, Hq, Hkv, Nq, Nk, causal, kpw, min_nw);
}

// Workspace of the backward pass: the (L2, D) pair of every query row,
// rounded up to 256 bytes, then (with the heads of a group split into parts)
// the parts' fp32 partial sums of dK and of dV.
size_t bwd_pairs_bytes(int B, int Hq, int Nq) { return ((size_t)B * Hq * Nq * 2 * sizeof(float) + 255) / 256 * 256; }
size_t bwd_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal) {
  const fa_kvplan_t pk = plan_bwd_dkdv(B, Hq, Hkv, Nq, Nk, d, causal);
  size_t n = bwd_pairs_bytes(B, Hq, Nq);
  if (pk.hsplit > 1) n += (size_t)2 * pk.hsplit * B * Hkv * (size_t)Nk * d * sizeof(float);
  return n;
}

}  // namespace

namespace fa {
// The forward entry points' host-side argument checks, for fa_noalloc.hip.
fa_status validate_forward(const void* q, const void* k, const void* v, const void* o, const void* lse, int B, int Hq,
                           int Hkv, int Nq, int Nk, int d, float scale, int causal) {
  return validate(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal);
}
}  // namespace fa

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
    case FA_ERR_WORKSPACE: return "workspace missing, too small or not 16-byte aligned";
    case FA_ERR_SCRATCH_LIMIT: return "the call needs more than the library's fixed scratch";
  }
  return "unknown status";
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Nq,
                 int Nk, int d, float scale, int causal, void* stream) {
  return forward(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, stream, 0);
}

fa_status fa_fwd_exp2_emulated(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                               int Hkv, int Nq, int Nk, int d, float scale, int causal, int quarters, void* stream) {
  const fa_status st = validate(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal);
  if (st != FA_OK) return st;
  if (d == 256) return FA_ERR_HEAD_DIM;  // its variants are built for d = 64 and 128
  if (quarters != 1 && quarters != 2) return FA_ERR_FLAG;
  return forward(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, stream, 0, quarters);
}

fa_status fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int Hq, int Hkv,
                     int Nq, int Nk, int d, float scale, int causal, void* stream) {
  return forward(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, stream, 1);
}

fa_status fa_fp8_prepare(const void* q, const void* k, const void* v, void* q8, void* k8, void* v8t, float* descale,
                         unsigned* amax_ws, const float* signs, float scale, int B, int Hq, int Hkv, int Nq, int Nk,
                         int d, void* stream) {
  if (!q || !k || !v || !q8 || !k8 || !v8t || !descale || !amax_ws) return FA_ERR_NULL;
  const fa_status st = validate_shape(B, Hq, Hkv, Nq, Nk, d);
  if (st != FA_OK) return st;
  if (fa::fp8_prepare_too_large(B, Hq, Hkv, Nq, Nk)) return FA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q8) || !aligned16(k8) || !aligned16(v8t) ||
      !aligned4(descale) || !aligned4(amax_ws) || (signs && !aligned4(signs)))
    return FA_ERR_ALIGN;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
  const float c0 = (float)((double)scale * LOG2E);
  const hipError_t e = fa::launch_fp8_prepare(q, k, v, q8, k8, v8t, descale, amax_ws, signs, c0, B, Hq, Hkv, Nq, Nk,
                                              d, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd_fp8(const void* q8, const void* k8, const void* v8t, const float* descale, void* o, float* lse, int B,
                     int Hq, int Hkv, int Nq, int Nk, int d, int causal, void* stream) {
  if (!q8 || !k8 || !v8t || !descale || !o) return FA_ERR_NULL;
  const fa_status st = validate_shape(B, Hq, Hkv, Nq, Nk, d);
  if (st != FA_OK) return st;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8t) || !aligned16(o) || (lse && !aligned16(lse)) ||
      !aligned4(descale))
    return FA_ERR_ALIGN;
  if (causal != 0 && causal != 1) return FA_ERR_FLAG;
  const fa_plan_t p = plan_for(B, Hq, Hkv, Nq, Nk, d, causal, KIND_FP8);
  if (p.nwg > 0x7fffffffLL) return FA_ERR_SHAPE;
  const hipError_t e = fa::launch_fwd_fp8(q8, k8, v8t, descale, o, lse, p, d, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_fwd_splitkv_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, int nsplit) {
  if (validate_shape(B, Hq, Hkv, Nq, Nk, d) != FA_OK || nsplit < 0 || (causal != 0 && causal != 1)) return 0;
  return splitkv_workspace_bytes(plan_splitkv(B, Hq, Hkv, Nq, Nk, d, causal, nsplit), d);
}

fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                         int Nq, int Nk, int d, float scale, int causal, int nsplit, void* workspace,
                         size_t workspace_bytes, void* stream) {
  fa_status st = validate(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal);
  if (st != FA_OK) return st;
  if (nsplit < 0) return FA_ERR_SHAPE;
  const fa_plan_t p = plan_splitkv(B, Hq, Hkv, Nq, Nk, d, causal, nsplit);
  if (p.nwg > 0x7fffffffLL) return FA_ERR_SHAPE;
  const float c = (float)((double)scale * LOG2E);
  if (p.nsplit <= 1) {
    const hipError_t e = fa::launch_fwd(q, k, v, o, lse, p, d, c, 0, nullptr, nullptr, (hipStream_t)stream);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
  }
  const size_t need = splitkv_workspace_bytes(p, d);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return FA_ERR_WORKSPACE;
  const long long rows = (long long)B * Hq * Nq;
  if (rows > 0x7fffffffLL) return FA_ERR_SHAPE;
  float* ows = (float*)workspace;
  float* lws = ows + (size_t)p.nsplit * rows * d;
  hipError_t e = fa::launch_fwd(q, k, v, nullptr, nullptr, p, d, c, 0, ows, lws, (hipStream_t)stream);
  if (e == hipSuccess) e = fa::launch_merge(ows, lws, o, lse, p.nsplit, rows, d, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal) {
  if (validate_shape(B, Hq, Hkv, Nq, Nk, d) != FA_OK || (causal != 0 && causal != 1)) return 0;
  return bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, causal);
}

namespace {

// Checks shared by the backward entry points (o and lse may be absent for
// the dK/dV stage, dq/dk/dv for the stage that does not write them).
fa_status validate_bwd(const void* const* ptrs, int nptrs, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                       int causal, const void* workspace, size_t workspace_bytes) {
  for (int i = 0; i < nptrs; ++i)
    if (!ptrs[i]) return FA_ERR_NULL;
  const fa_status st = validate_shape(B, Hq, Hkv, Nq, Nk, d);
  if (st != FA_OK) return st;
  for (int i = 0; i < nptrs; ++i)
    if (!aligned16(ptrs[i])) return FA_ERR_ALIGN;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
  if (causal != 0 && causal != 1) return FA_ERR_FLAG;
  // one query head's rows (the range of a buffer resource) fit in 31 bits
  if (((double)Nq + 64.0) * d * 4.0 >= 2147483648.0) return FA_ERR_SHAPE;
  if (workspace == nullptr || workspace_bytes < bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, causal) ||
      !aligned16(workspace))
    return FA_ERR_WORKSPACE;
  return FA_OK;
}

fa_status bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                 void* dq, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal, void* workspace,
                 size_t workspace_bytes, void* stream) {
  const void* ptrs[] = {q, k, v, o, dout, lse, dq};
  const fa_status st = validate_bwd(ptrs, 7, B, Hq, Hkv, Nq, Nk, d, scale, causal, workspace, workspace_bytes);
  if (st != FA_OK) return st;
  const fa_plan_t pq = plan_bwd_dq(B, Hq, Hkv, Nq, Nk, d, causal);
  if (pq.nwg > 0x7fffffffLL) return FA_ERR_SHAPE;
  const hipError_t e = fa::launch_bwd_dq(q, k, v, o, dout, lse, dq, (float*)workspace, pq, d,
                                         (float)((double)scale * LOG2E), scale, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dv, int B, int Hq,
                   int Hkv, int Nq, int Nk, int d, float scale, int causal, void* workspace, size_t workspace_bytes,
                   void* stream) {
  const void* ptrs[] = {q, k, v, dout, dk, dv};
  const fa_status st = validate_bwd(ptrs, 6, B, Hq, Hkv, Nq, Nk, d, scale, causal, workspace, workspace_bytes);
  if (st != FA_OK) return st;
  const fa_kvplan_t pk = plan_bwd_dkdv(B, Hq, Hkv, Nq, Nk, d, causal);
  if (pk.nwg > 0x7fffffffLL) return FA_ERR_SHAPE;
  float* part = pk.hsplit > 1 ? (float*)((char*)workspace + bwd_pairs_bytes(B, Hq, Nq)) : nullptr;
  const hipError_t e = fa::launch_bwd_dkdv(q, k, v, dout, dk, dv, (const float*)workspace, part, pk, d,
                                           (float)((double)scale * LOG2E), scale, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                    void* dq, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return bwd_dq(q, k, v, o, dout, lse, dq, B, Hq, Hkv, Nq, Nk, d, scale, causal, workspace, workspace_bytes, stream);
}

fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dv, int B,
                      int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return bwd_dkdv(q, k, v, dout, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale, causal, workspace, workspace_bytes, stream);
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                 void* workspace, size_t workspace_bytes, void* stream) {
  // both stages are validated before either is enqueued
  const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv};
  const fa_status st = validate_bwd(ptrs, 9, B, Hq, Hkv, Nq, Nk, d, scale, causal, workspace, workspace_bytes);
  if (st != FA_OK) return st;
  const fa_status s1 = bwd_dq(q, k, v, o, dout, lse, dq, B, Hq, Hkv, Nq, Nk, d, scale, causal, workspace,
                              workspace_bytes, stream);
  if (s1 != FA_OK) return s1;
  return bwd_dkdv(q, k, v, dout, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale, causal, workspace, workspace_bytes, stream);
}

size_t fa_mfma_ceiling_out_bytes(void) { return (size_t)fa::mfma_ceiling_workgroups() * 256 * sizeof(float); }

double fa_mfma_ceiling_flops(int fp8, int iters) { return iters < 1 ? 0.0 : fa::mfma_ceiling_flops(fp8 != 0, iters); }

fa_status fa_mfma_ceiling(float* out, size_t out_bytes, int fp8, int iters, int random, void* stream) {
  if (!out) return FA_ERR_NULL;
  if ((fp8 != 0 && fp8 != 1) || (random != 0 && random != 1)) return FA_ERR_FLAG;
  if (iters < 1) return FA_ERR_SHAPE;
  if (!aligned4(out) || out_bytes < fa_mfma_ceiling_out_bytes()) return FA_ERR_WORKSPACE;
  const hipError_t e = fa::launch_mfma_ceiling(out, fp8, iters, random, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_issue_cost_cases(void) { return fa::issue_cost_cases(); }

fa_status fa_issue_cost_case(int i, int* mfmas, int* exps, int* cvts, int* fmas) {
  if (!mfmas || !exps || !cvts || !fmas) return FA_ERR_NULL;
  return fa::issue_cost_case(i, mfmas, exps, cvts, fmas) ? FA_OK : FA_ERR_FLAG;
}

fa_status fa_issue_cost_case_mfma(int i, int* kind) {
  if (!kind) return FA_ERR_NULL;
  return fa::issue_cost_case_mfma(i, kind) ? FA_OK : FA_ERR_FLAG;
}

fa_status fa_issue_cost(float* out, size_t out_bytes, int i, int iters, void* stream) {
  if (!out) return FA_ERR_NULL;
  if (i < 0 || i >= fa::issue_cost_cases()) return FA_ERR_FLAG;
  if (iters < 1) return FA_ERR_SHAPE;
  if (!aligned4(out) || out_bytes < fa_mfma_ceiling_out_bytes()) return FA_ERR_WORKSPACE;
  const hipError_t e = fa::launch_issue_cost(out, i, iters, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"

// fa_noalloc.hip -- fa_fwd_splitkv_noalloc: the key-split forward pass with
// its workspace in a fixed array the library owns, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// `scratch` is one file-scope device array per GPU, FA_NOALLOC_SCRATCH_BYTES
// large, held until the process ends.  Host code never passes the array's
// name to a kernel (in host code it is a stand-in, not a device address):
// the first call on each device, with that device current, looks up the
// array's device address with hipGetSymbolAddress and keeps it; every launch
// then takes that address.  Nothing here allocates or frees.
//
// The scratch holds the parts' fp32 outputs and log-sum-exps between the
// attention kernel and the merge kernel; every element the merge reads is
// written first by the same call, so nothing needs clearing.  All calls on
// one GPU share the array: calls that overlap on one GPU (other streams,
// other host threads) race on it and must be ordered by the caller.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "fa.h"

namespace fa {
fa_status validate_forward(const void* q, const void* k, const void* v, const void* o, const void* lse, int B, int Hq,
                           int Hkv, int Nq, int Nk, int d, float scale, int causal);
}

namespace {

static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::once_flag g_once[MAX_DEVICES];
void* g_ptr[MAX_DEVICES];
hipError_t g_err[MAX_DEVICES];

// Device address of `scratch` on the current device (nullptr on failure).
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  return g_ptr[dev];
}

}  // namespace

extern "C" {

fa_status fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                                 int Hkv, int Nq, int Nk, int d, float scale, int causal, int nsplit, void* stream) {
  // argument checks on the host first (fa_fwd_splitkv's), then the size
  // check against the fixed scratch; nothing touches HIP before
  const fa_status st = fa::validate_forward(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal);
  if (st != FA_OK) return st;
  if (nsplit < 0) return FA_ERR_SHAPE;
  const size_t need = fa_fwd_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, causal, nsplit);
  if (need == 0)  // a plan without parts: fa_fwd's kernel, no workspace
    return fa_fwd_splitkv(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, nsplit, nullptr, 0, stream);
  if (need > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH_LIMIT;
  void* ws = scratch_address();
  if (ws == nullptr) return FA_ERR_HIP;
  return fa_fwd_splitkv(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, nsplit, ws,
                        (size_t)FA_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"

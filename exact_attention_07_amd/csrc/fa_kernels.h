// fa_kernels.h -- internal interface between the C-ABI layer and the kernels.
#ifndef FA_KERNELS_H
#define FA_KERNELS_H

#include <hip/hip_runtime.h>

#include "plan.h"

namespace fa {

// Query rows per wave of the forward kernel for head dimension d.
int queries_per_wave(int d, int f32);

// Workgroups of a persistent launch whose kernel fits per_cu workgroups on
// a CU: nwg, or per_cu per CU of the current device (the CU count rounded
// down to a multiple of 8) when nwg is larger; the kernel then takes its
// work items in rounds (fa_persistent_item).  The persistent forms and
// their workgroups per CU:
//   forward: 8 waves at d = 128 and 4 at d = 256 (one); causal 4 waves at
//     d = 64 and 128 (two);
//   fp8 forward: 4 waves at d = 256 (one); causal 4 waves at d = 64 and
//     128 (two);
//   dQ: 8 waves at d = 128, 4 at d = 256 up to Nq = 4096 (one); causal
//     4 waves at d = 128 up to Nq = 4096 (two);
//   dK/dV, up to Nq = 4096 with two items per workgroup: 8 waves at
//     d = 128, 4 waves at d = 64, 128 and 256 (one); causal 2 waves at
//     d = 64 (two).
unsigned persistent_grid(long long nwg, int per_cu = 1);

// CUs of the current device, rounded down to a multiple of 8 (one per XCD
// share); 0 if the runtime cannot say.  Read once per device.
int cu_count();

// The measured MFMA ceiling (fa_ceiling.hip): workgroups of the loop kernel
// (two per CU, four waves each), its matrix flops for `iters` rounds, and
// the launch (fp8: the e4m3 instruction; random: operands that change from
// instruction to instruction, else constant).  out: one float per thread,
// mfma_ceiling_workgroups() * 256 of them.
unsigned mfma_ceiling_workgroups();
double mfma_ceiling_flops(int fp8, int iters);
hipError_t launch_mfma_ceiling(float* out, int fp8, int iters, int random, hipStream_t stream);
// The issue-cost loop (fa_issue.hip): case i of issue_cost_cases() rounds
// of MFMAs with exponentials, e4m3 packings and FMAs beside them; the same
// grid and output size as the ceiling loop.
int issue_cost_cases();
bool issue_cost_case(int i, int* mfmas, int* exps, int* cvts, int* fmas);
// the case's matrix instruction: 0 bf16 32x32x16, 1 e4m3 32x32x64, 2 the
// same with E8M0 scale operands, 3 the two e4m3 forms alternating
bool issue_cost_case_mfma(int i, int* kind);
hipError_t launch_issue_cost(float* out, int i, int iters, hipStream_t stream);

// Enqueue the forward kernel.  c = scale * log2(e).  f32 selects fp32
// operands (split into bf16 hi/lo parts inside the kernel).  With a key
// split (p.nsplit > 1, bf16 only) the kernel writes the partial results of
// every range to ows ([nsplit][B][Hq][Nq][d] fp32) and lws ([nsplit][B][Hq][Nq]).
// emu (bf16, d = 64 and 128 only): 1 or 2 of every four exponentials on the
// FMA pipe (exp2_poly) instead of the exponential unit.
hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, const fa_plan_t& p, int d,
                      float c, int f32, float* ows, float* lws, hipStream_t stream, int emu = 0);

// Enqueue the merge of nsplit partial results of rows = B*Hq*Nq rows into o
// (bf16) and lse (fp32, may be NULL).
hipError_t launch_merge(const float* ows, const float* lws, void* o, float* lse, int nsplit, long long rows, int d,
                        hipStream_t stream);

// Enqueue the fp8 forward kernel (operands from launch_fp8_prepare, whose
// Q codes carry the softmax scale in log2 units).
hipError_t launch_fwd_fp8(const void* q8, const void* k8, const void* v8t, const float* descale, void* o, float* lse,
                          const fa_plan_t& p, int d, hipStream_t stream);

// True if a preparation of this shape needs a grid of 2^31 or more
// workgroups (such shapes are rejected).
bool fp8_prepare_too_large(int B, int Hq, int Hkv, int Nq, int Nk);

// Enqueue the fp8 preparation: optional Hadamard rotation of Q and K, Q
// multiplied by c0 = softmax scale * log2(e), per-tensor amax, e4m3
// quantisation (power-of-two scales for Q and K), V transposed (fa.h
// describes the layouts).  amax: 3 device words of workspace.
hipError_t launch_fp8_prepare(const void* q, const void* k, const void* v, void* q8, void* k8, void* v8t,
                              float* descale, unsigned* amax, const float* signs, float c0, int B, int Hq, int Hkv,
                              int Nq, int Nk, int d, hipStream_t stream);

// Backward pass: keys per wave and most waves per workgroup of the dK/dV
// kernel for head dimension d.
int bwd_keys_per_wave(int d);
int bwd_dkdv_max_waves(int d);

// Enqueue the dQ kernel of the backward pass (plan pq).  It also writes the
// per-row pairs (LSE log2 e, rowsum(dO o O)) into ld, [B][Hq][Nq][2] fp32.
// c = scale * log2(e).
hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, void* dq, float* ld, const fa_plan_t& pq, int d, float c, float scale,
                         hipStream_t stream);

// Enqueue the dK/dV kernel of the backward pass (plan pk); reads the pairs
// launch_bwd_dq wrote into ld.
// With pk.hsplit > 1 the partial sums of the head parts go to `part`
// (2 * hsplit * B * Hkv * Nk * d floats, 16-byte aligned) and a second kernel
// adds them into dK and dV.
hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dv,
                           const float* ld, float* part, const fa_kvplan_t& pk, int d, float c, float scale,
                           hipStream_t stream);

}  // namespace fa

#endif

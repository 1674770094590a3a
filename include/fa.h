/*
 * fa.h -- C ABI of libfa.so, fused exact-attention forward and backward passes for AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed (the definition on "FlashAttention (SV)", section
 * "Problematik med standard-attention"):
 *
 *     O   = softmax(scale * Q K^T) V            per (batch b, query head h)
 *     LSE = ln sum_j exp(scale * q_i . k_j)     natural log, scale included
 *
 * without ever writing the N x N score matrix to memory: Q, K and V are tiled
 * through on-chip memory, the softmax is computed online with a running row
 * maximum and a running sum of exponentials ("FlashAttention (SV)", sections
 * "Tiling och blockbearbetning" and "Online-beräkning av Softmax"), and one
 * kernel does Q K^T, masking, softmax and the product with V (section
 * "Sammanslagning av operationer").  The output rescaling that the online
 * softmax needs is skipped while the running maximum stays within 2^8 of the
 * value the exponentials were taken against ("FlashAttention-4震撼发布",
 * first of the two algorithmic improvements); the result is exact either way.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout: contiguous row-major tensors
 *     q, o : [B][Hq][Nq][d]        k, v : [B][Hkv][Nk][d]
 *     lse  : [B][Hq][Nq] float32   (may be NULL: then it is not written)
 * GQA/MQA ("FlashAttention-4震撼发布", FlashAttention-2 list): Hq must be a
 *     multiple of Hkv; query head h reads key/value head h / (Hq / Hkv).
 *     Hkv == Hq is ordinary multi-head attention, Hkv == 1 is MQA.
 * Head dimension d: 64, 128 or 256 (FlashAttention-2 list: head sizes up to
 *     256).
 * causal: 0 or 1.  With causal = 1 key j is visible to query i iff
 *     j <= i + (Nk - Nq) (bottom-right alignment; for Nq == Nk this is the
 *     usual lower triangle).  A query that sees no key gets O = 0 and
 *     LSE = -inf.
 * scale: finite and > 0 (usually 1/sqrt(d)).
 * Memory: every pointer is device memory owned by the caller, 16-byte
 *     aligned.  The library allocates, frees and synchronises nothing and
 *     keeps no per-call state; calls are asynchronous on `stream` (a
 *     hipStream_t, NULL = the default stream), so buffers must stay alive
 *     until the enqueued work is done.  Outputs must not overlap inputs.
 *     Calls are thread-safe.
 * Errors: argument errors are detected on the host before any HIP call and
 *     nothing is enqueued.  A failed launch returns FA_ERR_HIP.  Faults inside
 *     a kernel surface at the caller's next synchronisation.  No C++
 *     exception crosses this interface.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,       /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,      /* B, Hq, Hkv, Nq or Nk < 1, or a tensor too large to index */
  FA_ERR_HEAD_DIM = 3,   /* d not in {64, 128, 256} */
  FA_ERR_GQA_RATIO = 4,  /* Hq not a multiple of Hkv */
  FA_ERR_ALIGN = 5,      /* a pointer is not 16-byte aligned */
  FA_ERR_SCALE = 6,      /* scale not finite or not > 0 */
  FA_ERR_HIP = 7,        /* the HIP runtime refused the launch */
  FA_ERR_FLAG = 8,       /* causal not 0 or 1 */
  FA_ERR_WORKSPACE = 9,  /* workspace missing, too small or not 16-byte aligned */
  FA_ERR_SCRATCH_LIMIT = 10 /* the call needs more than the library's fixed scratch */
} fa_status;

/* Version of this interface; bumped on any incompatible change. */
#define FA_ABI_VERSION 2
int fa_abi_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* fa_status_string(fa_status s);

/*
 * bfloat16 forward pass.  q, k, v, o hold bf16 values; lse is float32.
 * Products are accumulated in fp32; the probabilities multiply V in bf16;
 * O is rounded to bf16 (nearest even).
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int Nq, int Nk, int d,
                 float scale, int causal, void* stream);

/*
 * fa_fwd with part of the exponentials computed on the FMA pipe instead of
 * the hardware exponential unit ("FlashAttention-4震撼发布：性能再攀新高",
 * second algorithmic improvement: a polynomial emulation of the exponential
 * for some of the scores, where the exponential unit is the bottleneck).
 * For `quarters` (1 or 2) of every four scores of a row, 2^x is formed as
 * p(f) * 2^n with x = n + f, n = floor(x), and p the cubic of largest
 * relative error 7.5e-5 on [0, 1) (csrc/fa_exp2_coef.h, fitted by
 * exact_attention_07_amd/exp2_fit.py); the others take v_exp_f32.  Masked
 * keys still weigh exactly 0.  The result equals fa_fwd's up to that error
 * in the probabilities.  On gfx950 the exponential unit does not limit the
 * kernel, so this variant is slower than fa_fwd (it exists to measure that
 * trade); fa_fwd remains the path to use.
 *   quarters  1 or 2, else FA_ERR_FLAG
 *   d         64 or 128 (FA_ERR_HEAD_DIM for 256)
 * Everything else as for fa_fwd (no key split).
 */
fa_status fa_fwd_exp2_emulated(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int Hq, int Hkv, int Nq, int Nk, int d,
                               float scale, int causal, int quarters, void* stream);

/*
 * float32 forward pass: q, k, v, o hold float32 values.  The operation is
 * fa_fwd's, the definition on "FlashAttention (SV)", section "Problematik
 * med standard-attention", computed by the same tiled, fused, online-softmax
 * method (sections "Tiling och blockbearbetning", "Online-beräkning av
 * Softmax", "Sammanslagning av operationer"); only the operand precision
 * differs.  The kernel splits every fp32 operand into a bf16 head and a bf16
 * tail (x = hi + lo, exact to about 2^-16 relative) and forms each product
 * from the three largest partial products on bf16 MFMA, so scores and the
 * output carry close to fp32 accuracy.  Arguments, layouts, ownership and
 * errors as for fa_fwd (16-byte aligned float32 tensors).
 */
fa_status fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                     int B, int Hq, int Hkv, int Nq, int Nk, int d,
                     float scale, int causal, void* stream);

/*
 * bfloat16 forward pass with the keys split into ranges, for grids too small
 * to fill the GPU (decoding with a few query rows over a long context, small
 * batches).  Each workgroup computes the attention of its rows over one key
 * range and writes that part's output (normalised by the part's own sum)
 * and log-sum-exp; a second kernel combines the parts exactly:
 *     LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s
 * ("FlashAttention (SV)", section "Online-beräkning av Softmax": the
 * statistics of separate blocks combine exactly).  Inputs, outputs and
 * conventions as for fa_fwd; the result equals fa_fwd's up to rounding.
 *
 *   nsplit     number of key ranges; 0 lets the library choose (enough
 *              workgroups to fill the GPU).  The ranges hold equal numbers
 *              of 64-key tiles (the last may be shorter), so the number used
 *              can be below the one asked for; 1 (or a choice of 1) runs
 *              fa_fwd's kernel and needs no workspace.
 *   workspace  device memory of at least fa_fwd_splitkv_workspace_size(...)
 *              bytes for the same arguments, 16-byte aligned, owned by the
 *              caller and not shared with a call in flight; holds the parts
 *              as float32 O [nsplit][B][Hq][Nq][d] followed by float32 LSE
 *              [nsplit][B][Hq][Nq].  May be NULL when the size is 0.
 * Errors: those of fa_fwd; FA_ERR_SHAPE for nsplit < 0 (or too many rows);
 * FA_ERR_WORKSPACE for a missing, small or misaligned workspace.
 */
size_t fa_fwd_splitkv_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, int nsplit);
fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                         int nsplit, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_fwd_splitkv without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The parts live in a fixed array of
 * FA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends; the call itself allocates and frees nothing.
 * Arguments, layouts, result and errors as for fa_fwd_splitkv, plus
 * FA_ERR_SCRATCH_LIMIT when fa_fwd_splitkv_workspace_size(...) for the same
 * arguments exceeds FA_NOALLOC_SCRATCH_BYTES (ask for fewer ranges, or use
 * fa_fwd_splitkv with a workspace).  Every call on one GPU uses that GPU's
 * array: calls that overlap on one GPU (on other streams or from other host
 * threads) race on it, so the caller orders them.
 */
#define FA_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)
fa_status fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                                 int nsplit, void* stream);

/*
 * FP8 preparation ("FlashAttention-3 — 闪电注意力-3", section on low
 * precision and the reduction of quantisation error): rotate Q and K by an
 * orthogonal matrix, quantise Q, K and V to 8-bit floating point with one
 * scale per tensor.
 *
 *   q, k, v   bf16, [B][Hq][Nq][d], [B][Hkv][Nk][d], [B][Hkv][Nk][d]
 *   signs     fp32, d values of +1 or -1 (device), or NULL: no rotation.
 *             Rotation: x -> x diag(signs) H_d / sqrt(d) for every row of Q
 *             and K, H_d the Sylvester Hadamard matrix (H_1 = [1],
 *             H_2n = [[H, H], [H, -H]]); V is not rotated.  The product
 *             Q K^T is unchanged by the rotation.
 *   scale     the softmax scale the codes are prepared for (finite, > 0;
 *             usually 1/sqrt(d)): Q is multiplied by c0 = scale * log2(e)
 *             before it is quantised, so that fa_fwd_fp8's score products
 *             come out in the base-2 units its exponentials take
 *   q8, k8    OCP E4M3 codes (1 byte each), same layouts as q and k
 *   v8t       E4M3 codes of V transposed: [B][Hkv][d][Nkp], Nkp = Nk rounded
 *             up to a multiple of 64.  Within each block of 64 keys, key
 *             kk = 32 a + 8 g + 4 h + r (a, h in {0,1}, g, r in {0..3}) is
 *             stored at position 32 h + 16 a + 4 g + r; keys >= Nk are zero.
 *   descale   3 fp32 (device): s_q, s_k, s_v.  s_q is the smallest power of
 *             two with amax|c0 x| / s_q <= 448 over the whole rotated Q
 *             (x = rotated query), and c0 x is represented by
 *             s_q * decode(code); s_k is the smallest power of two with
 *             amax|x| / s_k <= 448 over the whole rotated K; s_v =
 *             amax|V| / 448; x (rotated K, V) is represented by
 *             s * decode(code); s = 1 for an all-zero tensor.  Power-of-two
 *             s_q and s_k let the attention kernel apply them exactly through
 *             the matrix core's scale operands; in a floating-point format the
 *             choice of scale within a factor of two changes no code's
 *             relative precision.
 *   amax_ws   3 uint32 of device workspace (zeroed and used inside).
 * Codes are rounded to nearest even; |x| / s <= 448 by construction.  The
 * scales stay on the device: nothing is synchronised.  Pointers of the code
 * tensors and q, k, v are 16-byte aligned; descale, amax_ws, signs 4-byte.
 */
fa_status fa_fp8_prepare(const void* q, const void* k, const void* v, void* q8, void* k8, void* v8t,
                         float* descale, unsigned* amax_ws, const float* signs, float scale,
                         int B, int Hq, int Hkv, int Nq, int Nk, int d, void* stream);

/*
 * FP8 forward pass on the output of fa_fp8_prepare: O (bf16) and LSE (fp32)
 * of softmax(scale * Q K^T) V, with the scale given to fa_fp8_prepare (the
 * Q codes carry it) ("FlashAttention (SV)", section "Problematik
 * med standard-attention") with Q, K, V represented by their codes and
 * scales, both products on 8-bit floating-point matrix instructions
 * ("FlashAttention-3 — 闪电注意力-3", section on the Hopper GPU's new
 * hardware features: FP8 at twice the FP16 rate; section on low precision
 * and the reduction of quantisation error: Q and K rotated before
 * quantisation, which leaves Q K^T unchanged).  Both products run on e4m3
 * MFMA with fp32 accumulation; the probabilities multiply V as e4m3 values
 * (unscaled, at most 2^8), while the row sums and the LSE use the fp32
 * probabilities.  descale[0] and descale[1] must be powers of two (as
 * fa_fp8_prepare writes them; only their exponents are used).  Conventions
 * (GQA, causal, errors) as for fa_fwd.
 */
fa_status fa_fwd_fp8(const void* q8, const void* k8, const void* v8t, const float* descale,
                     void* o, float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                     int causal, void* stream);

/*
 * Backward pass (bfloat16): the gradients of L with respect to Q, K and V for
 * an upstream gradient dout = dL/dO of fa_fwd's output.  The pages report
 * the method's training speed-ups ("FlashAttention-4震撼发布",
 * FlashAttention-2 list; "FlashAttention (SV)", section "Empiriska
 * resultat") but print no backward algorithm; what is computed is the
 * derivative of the definition above, with P = softmax(scale Q K^T):
 *
 *     dV = P^T dO,   dP = dO V^T,   D_i = sum_c dO_ic O_ic,
 *     dS = P o (dP - D),   dQ = scale dS K,   dK = scale dS^T Q,
 *
 * per (b, query head); with GQA the gradients of a key/value head are summed
 * over the query heads that read it.  P is recomputed tile by tile from q, k
 * and the forward pass's lse (none of the N x N matrices reaches memory).
 *
 *   q, k, v    the forward pass's inputs (bf16, layouts as for fa_fwd)
 *   o, lse     its outputs: O (bf16) and the natural-log LSE (fp32), as
 *              fa_fwd wrote them for the same q, k, v, scale and causal
 *   dout       dL/dO, bf16, q's layout
 *   dq         out: dL/dQ, bf16, q's layout
 *   dk, dv     out: dL/dK, dL/dV, bf16, k's layout (every element written)
 *   workspace  device memory of at least fa_bwd_workspace_size(...) bytes,
 *              16-byte aligned, owned by the caller and not shared with a
 *              call in flight; its contents on entry do not matter.  It
 *              holds the per-row pair (LSE log2(e), D) between the two
 *              kernels (B * Hq * Nq * 8 bytes, rounded up to 256).  When a
 *              group has too few key blocks to fill the GPU (few key/value
 *              heads, G = Hq / Hkv > 1), the G query heads of each group are
 *              split into parts whose fp32 partial sums of dK and dV follow
 *              the pairs (2 * parts * B * Hkv * Nk * d * 4 bytes) and are
 *              added by a second kernel; fa_bwd_workspace_size includes them.
 * Products run on bf16 MFMA with fp32 accumulation; P and dS multiply in
 * bf16; the gradients are rounded to bf16 (nearest even).  D is formed from
 * the bf16 O.  Rows that see no key (LSE = -inf) contribute nothing.
 * Errors: those of fa_fwd (every pointer except the workspace required);
 * FA_ERR_WORKSPACE for a missing, small or misaligned workspace.  fa_bwd
 * checks every argument before it enqueues anything.
 * fa_bwd_workspace_size returns 0 for arguments fa_bwd would reject.
 *
 * fa_bwd runs two kernels in stream order, also available on their own:
 *   fa_bwd_dq    dq, plus the per-row pairs (LSE log2(e), D) into the
 *                workspace ([B][Hq][Nq][2] float32);
 *   fa_bwd_dkdv  dk and dv; reads those pairs (and writes the partial
 *                sums, if any, after them), so it must follow an fa_bwd_dq
 *                with the same arguments and workspace (on the same stream,
 *                or after it has completed).
 * fa_bwd(...) is fa_bwd_dq(...) followed by fa_bwd_dkdv(...).
 */
size_t fa_bwd_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal);
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv,
                 int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                 void* workspace, size_t workspace_bytes, void* stream);
fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                    float scale, int causal, void* workspace, size_t workspace_bytes, void* stream);
fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dv,
                      int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Measurement helper, not part of the attention computation: the measured
 * MFMA ceiling.  The pages state attention throughput as a share of the
 * GPU's peak matrix rate ("FlashAttention-3 — 闪电注意力-3", section
 * "性能与意义": 75-85 % of H100's peak; "FlashAttention (SV)", section
 * "FlashAttention-2 (2023)": 50-73 % of A100's).  On MI355X the sustained
 * clock under a dense matrix load is set by the power limit and by how much
 * the operand bits toggle, so the nominal peak is not reachable by any
 * kernel; this call runs a loop of nothing but the matrix instructions the
 * attention kernels use (v_mfma_f32_32x32x16_bf16, or with fp8 = 1
 * v_mfma_f32_32x32x64_f8f6f4), two waves per SIMD on every CU, so that the
 * rate it reaches, timed by the caller, is the ceiling for matrix work at
 * the clock the chip sustains at that moment.
 *
 *   out        device memory for one float per thread of the loop, at least
 *              fa_mfma_ceiling_out_bytes() bytes, 4-byte aligned (the sums are
 *              stored only so that no work is optimised away)
 *   fp8        0: bf16 instruction, 1: e4m3 instruction
 *   iters      rounds of 16 matrix instructions per wave, >= 1
 *   random     1: operands that change from instruction to instruction
 *              (pseudo-random values, the toggling of real data); 0: constant
 *   fa_mfma_ceiling_flops(fp8, iters) gives the matrix flops of one launch.
 * Errors: FA_ERR_NULL (out), FA_ERR_WORKSPACE (out_bytes too small or out
 * misaligned), FA_ERR_SHAPE (iters < 1), FA_ERR_FLAG (fp8 or random not 0/1),
 * FA_ERR_HIP (launch).
 */
size_t fa_mfma_ceiling_out_bytes(void);
double fa_mfma_ceiling_flops(int fp8, int iters);
fa_status fa_mfma_ceiling(float* out, size_t out_bytes, int fp8, int iters, int random, void* stream);

/*
 * Measurement helper, not part of the attention computation: the cost of
 * vector work beside the matrix core.  "FlashAttention-4震撼发布：性能再攀新高"
 * (second algorithmic improvement) computes part of the exponentials with a
 * polynomial on the FMA units because on its GPU the exponential unit is
 * the narrow one.  Whether that can pay depends on what an exponential
 * costs against an FMA when both sit beside matrix work.  Case i is a loop
 * whose rounds hold `mfmas` MFMAs of the case's kind (random operands),
 * `exps` v_exp_f32, `cvts` v_cvt_pk_fp8_f32 and `fmas` v_fma_f32 per wave,
 * spread evenly, two waves per SIMD on every CU; the caller times launches
 * of each case against the MFMA-only case of the same kind.  The kinds:
 * 0 v_mfma_f32_32x32x16_bf16, 1 v_mfma_f32_32x32x64_f8f6f4 on e4m3,
 * 2 the same with E8M0 scale operands (both 2^0), 3 kinds 2 and 1
 * alternating (the fp8 kernel's S and P V products).  The cases include the
 * bf16 and fp8 kernels' mixes per four bf16 MFMAs, each also with a quarter
 * and with half of its exponentials replaced by seven fast instructions,
 * and the fp8 kernel's mix per two of its own MFMAs.
 *
 *   fa_issue_cost_cases()     number of cases
 *   fa_issue_cost_case(i, …)  the case's per-round counts (FA_ERR_NULL for a
 *                             null pointer, FA_ERR_FLAG for i out of range)
 *   fa_issue_cost_case_mfma(i, kind)  the case's MFMA kind (same errors)
 *   out, out_bytes            as for fa_mfma_ceiling
 *   iters                     rounds per wave, >= 1
 * Errors: FA_ERR_NULL (out), FA_ERR_FLAG (i out of range), FA_ERR_SHAPE
 * (iters < 1), FA_ERR_WORKSPACE (out_bytes too small or out misaligned),
 * FA_ERR_HIP (launch).
 */
int fa_issue_cost_cases(void);
fa_status fa_issue_cost_case(int i, int* mfmas, int* exps, int* cvts, int* fmas);
fa_status fa_issue_cost_case_mfma(int i, int* kind);
fa_status fa_issue_cost(float* out, size_t out_bytes, int i, int iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */

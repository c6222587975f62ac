/*
 * fa_stable.h -- C ABI of a BF16 (and FP16) FlashAttention forward/backward library for AMD
 * MI355X (gfx950), with the stabilised safe-softmax shift for repeated row maxima.
 *
 * Operations (pages cited by title/address and section):
 *   - forward: the tiled online softmax of the BF16 Flash Attention article
 *     (ijyty.com/news/896914) §2.1 -- S = scale * Q K^T per block, running max m and running sum l,
 *     P^ = exp(S - m), O accumulated as diag(exp(m_prev - m)) O + P^ V, final O = diag(l)^-1 O --
 *     with the mixed-precision schedule of "Flash Attention低精度训练稳定性优化实践"
 *     (jsqmd.com/news/761560) §3.2 (fp32 accumulation of Q K^T, fp32 softmax, bf16 P^ V product)
 *     and the saved logsumexp of its §3.3;
 *   - stabilised shift: the repeated-maximum detection and conditional shift of the same article
 *     §4.1 (and "為什么BF16的FlashAttention會把訓練「炸掉」？", web578.cn, mechanism 2): with a
 *     repeated row maximum rm, m = beta * rm when rm > 0 and m = 0 when rm < 0;
 *   - backward: recomputation of P from the saved logsumexp ("FlashAttention 训练时为什么会梯度爆炸",
 *     cnnetsun.cn/a/2497354, §2), delta = rowsum(dO o O) (ijyty.com article §3.1), then dQ, dK, dV.
 *
 * Conventions shared by every entry point:
 *   - q, k, v, o, dO, dq, dk, dv: device pointers to contiguous [B, H, N, d] bfloat16 tensors
 *     (row-major, d fastest), 16-byte aligned.  bfloat16 is passed as raw 16-bit storage.
 *     fa_fwd_elem / fa_bwd_elem also take IEEE binary16 (FA_ELEM_F16) in the same layout.
 *   - lse, delta workspace: device pointers to contiguous [B, H, N] float32, 4-byte aligned.
 *     lse holds the natural-log logsumexp of the scaled scores: LSE = m + ln(l).
 *   - dupcnt, ones: device pointers to contiguous [B, H, N] int32, 4-byte aligned.
 *   - B, H, N >= 0 (an empty problem, B*H*N == 0, is a successful no-op); d is 64 or 128.
 *     N need not be a multiple of any tile size.  B*H*N*d < 2^40 and N*d*2 < 2^31 (one head
 *     spans less than 2 GiB).
 *   - causal: 0 or 1; causal masking is top-left aligned (key j is visible to query i iff j <= i).
 *   - scale: the score scale (typically 1/sqrt(d)), finite and > 0.
 *   - beta: the shift factor for positive repeated maxima, finite and >= 1 (1.25 recommended by
 *     the ijyty.com article §3.2).
 *   - stable_flag: 0 = standard safe softmax (m = running max);
 *                  1 = the pages' tie-conditional rule, applied per key block from the running
 *                      (max, repeat count) merged across blocks;
 *                  2 = tie-anticipating rule: the same shift applied whether or not a repeat has
 *                      been seen yet, so no unnormalised probability at a positive or negative
 *                      maximum can round to exactly 1.0.
 *     O, LSE and the gradients do not depend on stable_flag (the shift cancels on normalising).
 *   - stream: a hipStream_t (NULL = the default stream).  Every call is asynchronous on it.
 *
 * Ownership and behaviour: the caller allocates every buffer; the library never allocates, frees
 * or synchronises, keeps no per-call state and may be called from several threads.  Outputs are
 * overwritten, never accumulated into.  Every argument is validated before any HIP call; invalid
 * arguments return an error status and launch nothing.  A HIP failure returns FA_ERR_HIP and the
 * raw hipError_t value is available from fa_last_hip_error() on the calling thread.  Nothing is
 * thrown across the ABI.
 */
#ifndef FA_STABLE_H
#define FA_STABLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,    /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,   /* B, H or a sequence length negative, or the problem too large */
  FA_ERR_HEADDIM = 3, /* d is not 64 or 128 */
  FA_ERR_PARAM = 4,   /* causal, scale, beta, stable_flag, flags, stages or elem out of range */
  FA_ERR_ALIGN = 5,   /* a pointer is not aligned as stated above */
  FA_ERR_HIP = 6,     /* a HIP call failed; see fa_last_hip_error() */
  FA_ERR_SCRATCH = 7  /* fa_bwd_noalloc only: the problem needs more rows than its scratch holds */
} fa_status;

/* Forward pass: writes o [B,H,N,d] bf16 and lse [B,H,N] fp32.  Same as fa_fwd_ex with
 * dupcnt = ones = NULL. */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, int causal, float scale, float beta, int stable_flag,
           void* stream);

/* Forward pass with optional per-row diagnostics (either pointer may be NULL; when either is
 * non-NULL a variant of the kernel that also counts them runs):
 *   dupcnt[b,h,i] = number of visible keys j whose score equals the row maximum, i.e.
 *                   rowsum(S == rowmax(S)) of the ijyty.com article §4.1 / §7.1, computed on the
 *                   kernel's fp32 dot products;
 *   ones[b,h,i]   = number of visible keys whose unnormalised probability P^, as rounded to bf16
 *                   for the P^ V product, equals exactly 1.0.  It depends on the key-block width
 *                   returned by fa_fwd_kv_block(d, causal), since the shift is chosen per key block from
 *                   the running (max, count), and key blocks are processed in ascending order. */
int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
              int32_t* dupcnt, int32_t* ones,
              int B, int H, int N, int d, int causal, float scale, float beta, int stable_flag,
              void* stream);

/* Forward pass with training monitors and a numerics option (every diagnostic pointer may be
 * NULL; when any is non-NULL the diagnostics variant of the kernel runs):
 *   dupcnt, ones  as for fa_fwd_ex;
 *   smin[b,h,i]   = min over visible keys j of the scaled score S_ij = scale q_i.k_j, and
 *   smax[b,h,i]   = max over visible keys of S_ij: the range of the softmax input that
 *                   "Flash Attention低精度训练稳定性优化实践" (jsqmd.com/news/761560) §5 says to
 *                   monitor besides NaNs, fp32 [B,H,N].
 * flags: 0, or FA_FWD_COMPENSATED_SUM: the row sum l of the unnormalised probabilities is kept
 *   with a compensated (Kahan) running sum across key blocks, which the ijyty.com article §7.2
 *   recommends for the softmax denominator of large models; O and lse then use that sum.
 *   Other bits -> FA_ERR_PARAM.
 * fa_fwd_ex(...) == fa_fwd_stats(..., dupcnt, ones, NULL, NULL, ..., 0, stream). */
#define FA_FWD_COMPENSATED_SUM 1
int fa_fwd_stats(const void* q, const void* k, const void* v, void* o, float* lse,
                 int32_t* dupcnt, int32_t* ones, float* smin, float* smax,
                 int B, int H, int N, int d, int causal, float scale, float beta, int stable_flag,
                 int flags, void* stream);

/* Forward pass over Nq queries and Nk keys per head (every other convention as above):
 *   q, o        [B,H,Nq,d] bf16;  k, v [B,H,Nk,d] bf16;  lse and every diagnostic [B,H,Nq];
 *   causal      FA_CAUSAL_NONE (0), FA_CAUSAL_TOP_LEFT (1: key j visible to query i iff j <= i)
 *               or FA_CAUSAL_BOTTOM_RIGHT (2: iff j <= i + Nk - Nq, so the last query sees every
 *               key, the alignment of a query block appended to a longer key sequence);
 *   Nq, Nk >= 0, each independently ragged (no tile multiple needed).
 * The tile boundaries at the sequence ends follow the ijyty.com article §4.2 (a block's extent is
 * clipped to what is left of the sequence); a query block attending to a longer key sequence is
 * the generation setting its §6.1 extends the method to.  A query that sees no key (Nk == 0, or
 * bottom-right with i < Nq - Nk) gets O = 0, lse = -inf, dupcnt = ones = 0, smin = +inf,
 * smax = -inf.  With Nq == Nk both causal alignments equal fa_fwd_stats's causal = 1.
 * Empty problems (B*H == 0 or Nq == 0) are no-ops; k and v may be NULL when Nk == 0.
 * Errors as fa_fwd_stats; causal outside 0..2 -> FA_ERR_PARAM. */
#define FA_CAUSAL_NONE 0
#define FA_CAUSAL_TOP_LEFT 1
#define FA_CAUSAL_BOTTOM_RIGHT 2
int fa_fwd_qk(const void* q, const void* k, const void* v, void* o, float* lse,
              int32_t* dupcnt, int32_t* ones, float* smin, float* smax,
              int B, int H, int Nq, int Nk, int d, int causal, float scale, float beta,
              int stable_flag, int flags, void* stream);

/* Backward pass: from q, k, v, the forward's o and lse, and the upstream gradient dO, writes
 * dq, dk, dv [B,H,N,d] bf16.  delta_ws is a caller-owned fp32 workspace of
 * fa_bwd_workspace_bytes(B,H,N,d) bytes; on return (in stream order) it holds
 * delta = rowsum(dO o O) per row.  beta and stable_flag are validated like the forward's but do
 * not change the result: P is rebuilt from lse, which does not depend on the shift. */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dO, void* dq, void* dk, void* dv, float* delta_ws,
           int B, int H, int N, int d, int causal, float scale, float beta, int stable_flag,
           void* stream);

/* Backward pass restricted to a subset of its stages, in this order when several are set:
 *   FA_BWD_DELTA (1): delta_ws = rowsum(dO o O);
 *   FA_BWD_DKDV  (2): dk, dv (reads delta_ws);
 *   FA_BWD_DQ    (4): dq (reads delta_ws).
 * When FA_BWD_DELTA and FA_BWD_DQ are both set, the dQ kernel forms delta itself (same definition,
 * fp32, summed in another order, so values may differ from the delta kernel's in the last bits),
 * stores it in delta_ws and runs before dK/dV; the separate delta kernel is not launched.
 * fa_bwd == fa_bwd_ex(..., FA_BWD_ALL, stream).  Without FA_BWD_DELTA the caller guarantees that
 * delta_ws already holds delta for these o and dO (e.g. from an earlier call).  Pointers of
 * outputs whose stage is not selected are still validated.  stages outside 1..7 -> FA_ERR_PARAM. */
#define FA_BWD_DELTA 1
#define FA_BWD_DKDV 2
#define FA_BWD_DQ 4
#define FA_BWD_ALL 7
int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dO, void* dq, void* dk, void* dv, float* delta_ws,
              int B, int H, int N, int d, int causal, float scale, float beta, int stable_flag,
              int stages, void* stream);

/* Backward pass over Nq queries and Nk keys per head, as fa_bwd_ex with the shapes and causal
 * alignments of fa_fwd_qk: dq, dO, o [B,H,Nq,d]; dk, dv [B,H,Nk,d]; lse, delta_ws [B,H,Nq].  A
 * query that sees no key contributes nothing (its dq row is 0); a key that no query sees gets
 * dk = dv = 0.  No-op when B*H == 0 or Nq == Nk == 0.  Pointers of tensors with no elements
 * (the Nk-sized ones when Nk == 0, the Nq-sized ones when Nq == 0) may be NULL. */
int fa_bwd_qk(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dO, void* dq, void* dk, void* dv, float* delta_ws,
              int B, int H, int Nq, int Nk, int d, int causal, float scale, float beta,
              int stable_flag, int stages, void* stream);

/* Element type of the 16-bit tensors (q, k, v, o, dO, dq, dk, dv) for fa_fwd_elem / fa_bwd_elem:
 *   FA_ELEM_BF16 (0): bfloat16, the type every other entry point takes;
 *   FA_ELEM_F16  (1): IEEE binary16.
 * "Flash Attention低精度训练稳定性优化实践" (jsqmd.com/news/761560) §2.1 and §3.2 name both 16-bit
 * formats for the attention inputs and the P V product: fp16 keeps 11 significant bits against
 * bf16's 8 but tops out at 65504, so a score whose exponential exceeds it (e^12 ~ 1.63e5 already
 * does, "FlashAttention 训练时为什么会梯度爆炸", cnnetsun.cn/a/2497354, §3.1) overflows unless the
 * exponent is shifted first.  Every product still accumulates in fp32 and the softmax runs in fp32;
 * with either element type the unnormalised probabilities P^ = exp(S - m) are at most 1 after the
 * shift (P^ = 1 at a maximum only where m equals it), so they and P are in range, and they are
 * rounded (to nearest even) to the element type for the P^ V, P^T dO and dS products.  Where the
 * rule's shift leaves the largest P^ of a row below 2^-13 (a repeated maximum rm with
 * (beta - 1) rm > 13 ln 2, or a negative one below -13 ln 2, shifted to 0), the forward takes its
 * exponentials against m lowered by a whole number of binades so that the largest value lands in
 * (2^-14, 2^-13]: the common power of two cancels in O / l and in LSE, the rounding is unchanged
 * in relative terms, and P^ neither goes subnormal in fp16 nor rounds to 1.0.  The exact-1.0 count
 * (ones) compares the element type's 1.0. */
#define FA_ELEM_BF16 0
#define FA_ELEM_F16 1

/* fa_fwd_qk with the element type as an argument: fa_fwd_qk(...) ==
 * fa_fwd_elem(..., flags, FA_ELEM_BF16, stream).  elem outside {0, 1} -> FA_ERR_PARAM. */
int fa_fwd_elem(const void* q, const void* k, const void* v, void* o, float* lse,
                int32_t* dupcnt, int32_t* ones, float* smin, float* smax,
                int B, int H, int Nq, int Nk, int d, int causal, float scale, float beta,
                int stable_flag, int flags, int elem, void* stream);

/* fa_bwd_qk with the element type as an argument: fa_bwd_qk(...) ==
 * fa_bwd_elem(..., stages, FA_ELEM_BF16, stream).  lse and delta_ws stay fp32.  elem outside
 * {0, 1} -> FA_ERR_PARAM. */
int fa_bwd_elem(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dO, void* dq, void* dk, void* dv, float* delta_ws,
                int B, int H, int Nq, int Nk, int d, int causal, float scale, float beta,
                int stable_flag, int stages, int elem, void* stream);

/* fa_fwd_elem with one more per-row output (NULL allowed):
 *   mshift[b,h,i] = the shift m of the repeated-maximum rule after the last key block, fp32, in
 *                   the natural-log units of the scaled scores S: with rm the row maximum of S,
 *                   m = beta * rm when rm > 0 and rm repeats, m = 0 when rm < 0 and rm repeats, and
 *                   m = rm otherwise (the ijyty.com article §4.1 and its closed form in §3.2;
 *                   "為什么BF16的FlashAttention會把訓練「炸掉」？", web578.cn, mechanism 2).  With
 *                   stable_flag 0, m = rm; with 2 every row counts as repeating.  The value is the
 *                   kernel's own (formed from its running maximum and repeat test as each key block
 *                   forms it), -inf for a row that sees no key.  Writing it does not select the
 *                   diagnostics variant: with only mshift requested, the kernel that fa_fwd runs writes it.
 * fa_fwd_elem(...) == fa_fwd_diag(..., mshift = NULL, ...).  Errors as fa_fwd_elem. */
int fa_fwd_diag(const void* q, const void* k, const void* v, void* o, float* lse,
                int32_t* dupcnt, int32_t* ones, float* smin, float* smax, float* mshift,
                int B, int H, int Nq, int Nk, int d, int causal, float scale, float beta,
                int stable_flag, int flags, int elem, void* stream);

/* Forward pass with the P^ V product in FP8 (OCP E4M3, the "e4m3fn" encoding, largest value 448):
 * the lower-precision extension the ijyty.com article §6.1 names, with dynamic scaling.  Tensors,
 * shapes, diagnostics, causal alignments and errors as fa_fwd_qk (bf16 q, k, v, o); the scores
 * Q K^T, the softmax statistics, l and lse stay as in the bf16 forward.  Only the operands of the
 * P^ V product are rounded to E4M3 (round to nearest even):
 *   - V, per head and block of 128 consecutive keys: s = amax |V_block| / 448 (fp32; s = 1 for an
 *     all-zero block), each value stored as E4M3(v * (1 / s)) and standing for that value times s;
 *   - P^ = exp(S - m) <= 1, as E4M3(2^8 P^) (so that P^ down to 2^-14 keeps 4 significant bits),
 *     standing for that value times 2^-8.  Where the rule's shift leaves the largest P^ of the row
 *     below 2^-5 (see FA_ELEM_F16), P^ is first multiplied by the power of two 2^k that brings that
 *     largest value into (2^-6, 2^-5], and the product carries 2^-k (cancelling in O / l).
 * O = sum over blocks of the rescaled products, divided by the unrounded l.  ones counts the P^
 * whose rounded value is exactly 1.0 (2^8 P^ rounds to 256, i.e. P^ >= 0.96875).  The key blocks
 * of this forward are 128 keys wide whether or not it is causal.
 * workspace: caller-owned device memory of fa_fwd_fp8pv_workspace_bytes(B, H, Nk, d) bytes, 16-byte
 * aligned (may be NULL when Nk == 0); the call overwrites it with the E4M3 V blocks and their
 * scales, so concurrent calls need separate workspaces.  Two kernels run in order on the stream.
 * The backward of this forward is fa_bwd_qk (it rebuilds P from lse, which is unrounded). */
int fa_fwd_fp8pv(const void* q, const void* k, const void* v, void* o, float* lse,
                 int32_t* dupcnt, int32_t* ones, float* smin, float* smax, void* workspace,
                 int B, int H, int Nq, int Nk, int d, int causal, float scale, float beta,
                 int stable_flag, int flags, void* stream);

/* Bytes of the fa_fwd_fp8pv workspace: B*H*ceil(Nk/128)*(d*128 + 4) (0 for invalid shapes). */
size_t fa_fwd_fp8pv_workspace_bytes(int B, int H, int Nk, int d);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): fa_bwd without the delta workspace argument.  delta
 * lives in scratch memory inside the library, one static array per GPU holding
 * fa_bwd_noalloc_max_rows() fp32 values (2^21, 8 MiB), allocated with the library's code object
 * and held until the process ends; this call allocates, frees and synchronises nothing.  Every
 * call on one GPU shares that GPU's array: calls that overlap on one GPU (several streams, several
 * threads) race on it and must be serialised by the caller.  The array keeps the last call's
 * contents; nothing in it needs to start at zero (delta is written for every row before it is
 * read).  Results equal fa_bwd's bit for bit.  Errors as fa_bwd; B*H*N larger than
 * fa_bwd_noalloc_max_rows() -> FA_ERR_SCRATCH (nothing launched).  The array used is that of the
 * GPU the stream belongs to (the current device for the default stream); the first call for each
 * GPU looks up its address (HIP calls, no allocation), with that GPU made current for the lookup
 * and the caller's current device restored. */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dO, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, int causal, float scale, float beta, int stable_flag,
                   void* stream);
size_t fa_bwd_noalloc_max_rows(void);

/* Bytes of the delta workspace fa_bwd needs: B*H*N*4 (0 for invalid or empty shapes); for
 * fa_bwd_qk pass N = Nq. */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/* Width of the key blocks the forward processes per step for head dimension d and the given
 * causal flag (any non-zero alignment counts as causal; 0 if d is not supported): the
 * granularity at which the running maximum, repeat count and shift change. */
int fa_fwd_kv_block(int d, int causal);

/* Static, human-readable name of a status code. */
const char* fa_status_str(int status);

/* Raw hipError_t of the last FA_ERR_HIP returned on the calling thread (0 if none). */
int fa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_STABLE_H */

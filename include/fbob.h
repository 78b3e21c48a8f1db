/*
 * fbob.h - C ABI of the MI355X (gfx950) library for exact backward-over-backward
 * (BoB) of softmax attention.
 *
 * Method: "FlashBoB: I/O-Efficient Exact Backward-over-Backward for Softmax
 * Attention" (papernotes.org notes and abstract).  For one attention head with
 * S = tau Q K^T, P = softmax_row(S), O = P V and upstream gradient dO, the first
 * backward gives dQ, dK, dV ("FlashAttention 的反向传播设计", section 一).  BoB
 * differentiates the scalar
 *        Phi = <dQ, U_Q> + <dK, U_K> + <dV, U_V>
 * with respect to (Q, K, V, dO) and returns (dQ~, dK~, dV~, ddO~) plus the two
 * row scalars alpha_i = sum_j P_ij F_ij (F = tau (U_Q K^T + Q U_K^T)) and
 * E_i = sum_j P_ij dP~_ij (FlashBoB notes, "整体框架" and "关键设计" item 1).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  * All tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates nothing and keeps no state between calls (fbob_bob_ws takes its
 *    scratch memory from the caller as well).
 *  * Shapes: per-query-head tensors are [B, Hq, N, d] and per-key/value-head
 *    tensors are [B, Hkv, N, d], contiguous, d fastest.  Row vectors (L, D,
 *    alpha, E) are [B, Hq, N].  Hq must be a multiple of Hkv (grouped-query
 *    attention shares one K/V head among Hq/Hkv consecutive query heads).
 *  * dtype (fbob_dtype) is the storage type of the seven inputs Q, K, V, dO,
 *    U_Q, U_K, U_V.  O, L, D and every output are float32.  Arithmetic: bf16
 *    inputs use bf16 x bf16 -> fp32 MFMA; f32 inputs use fp32 MFMA; exp and all
 *    row scalars are fp32.
 *  * tau is the score scale (S = tau Q K^T); L is the natural-log log-sum-exp
 *    of the scaled scores of each row.
 *  * causal != 0 masks key positions j > i (P_ij = 0).
 *  * d must be 64 or 128.  N may be any value >= 0 (ragged tails are masked).
 *    B, Hq, Hkv or N equal to 0 is an empty problem: FBOB_OK, nothing written.
 *  * Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  Every output element is written exactly once (no atomics, no
 *    accumulate-into), so outputs need no initialisation.  Calls are reentrant.
 *  * Errors: arguments are validated before any HIP call and reported by the
 *    return value; the library never aborts, throws or prints.
 *      FBOB_ERR_INVALID_ARG  negative size, NULL pointer, bad dtype, Hq % Hkv,
 *                            non-finite or non-positive tau
 *      FBOB_ERR_UNSUPPORTED  d not 64 or 128, or a size that overflows int32
 *                            per-head indexing
 *      FBOB_ERR_ALIGNMENT    a pointer not 16-byte aligned
 *      FBOB_ERR_ALIAS        an output range overlaps an input or another output
 *      FBOB_ERR_HIP          a HIP launch error (hipGetLastError after launch; an
 *                            error the calling thread left pending before the call is
 *                            taken first and never reported; fbob_hip_error_string
 *                            names the HIP error)
 *      FBOB_ERR_SCRATCH      fbob_bob_noalloc only: the problem's split schedule
 *                            needs more than FBOB_SCRATCH_BYTES
 */
#ifndef FBOB_H_
#define FBOB_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FBOB_VERSION 1

typedef enum {
  FBOB_OK = 0,
  FBOB_ERR_INVALID_ARG = 1,
  FBOB_ERR_UNSUPPORTED = 2,
  FBOB_ERR_ALIGNMENT = 3,
  FBOB_ERR_ALIAS = 4,
  FBOB_ERR_HIP = 5,
  FBOB_ERR_SCRATCH = 6
} fbob_status;

/* Size of the static per-device scratch array used by fbob_bob_noalloc. */
#define FBOB_SCRATCH_BYTES ((int64_t)128 << 20)

typedef enum { FBOB_DTYPE_F32 = 0, FBOB_DTYPE_BF16 = 1 } fbob_dtype;

/*
 * Forward pass with the row state that BoB recomputes from.
 * FlashAttention blog, section 一 (S, P, O) and section 二 (keep per-row
 * statistics instead of P); FlashBoB notes, "关键设计" 1 (D_i = do_i^T o_i) and
 * "关键设计" 2 (P is rebuilt on chip from the stored log-partition L).
 *
 *   in : Q [B,Hq,N,d], K, V [B,Hkv,N,d], dO [B,Hq,N,d]   (dtype)
 *   out: O [B,Hq,N,d] = P V (fp32)
 *        L [B,Hq,N]   = log sum_j exp(tau Q_i . K_j)     (fp32, natural log)
 *        D [B,Hq,N]   = dO_i . O_i                        (fp32, from fp32 O)
 * dO and D may both be NULL: then only O and L are computed (the attention
 * forward alone); exactly one of them NULL is FBOB_ERR_INVALID_ARG.
 */
int fbob_forward(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                 float tau, int causal,
                 const void* Q, const void* K, const void* V, const void* dO,
                 float* O, float* L, float* D, void* stream);

/*
 * Device workspace, in bytes, that fbob_forward_ws can use for this problem (0 when the
 * row tiles fill the GPU, or the inputs are fp32: then fbob_forward_ws is fbob_forward).
 * Same size arguments as fbob_forward; writes the size to *bytes.  FBOB_ERR_INVALID_ARG
 * if bytes is NULL; size errors as fbob_forward.  No HIP call.
 */
int fbob_forward_workspace_size(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                                int64_t d, float tau, int causal, int64_t* bytes);

/*
 * fbob_forward with a caller-owned device workspace for problems too small to fill the
 * GPU: a work-group owns 256 query rows; when there are fewer of them than the resident
 * work-group slots (512 at d = 64, 256 at d = 128), each row tile's key sweep is split
 * over 2-16 work-groups.  Each keeps the online-softmax state of its keys (unnormalised
 * O, row sum, reference maximum) in fp32 in the workspace, and a reduction merges the
 * parts in a fixed order (FlashAttention blog, section 一: the softmax of a concatenation
 * from the blocks' maxima and sums) and writes O, L and D once.  Deterministic; the
 * results differ from fbob_forward's only by fp32 rounding order.  bf16 inputs.
 *   workspace       DEVICE pointer, 16-byte aligned, owned by the caller, at least
 *                   fbob_forward_workspace_size() bytes; NULL (or fewer bytes) runs
 *                   exactly fbob_forward.  Contents on entry ignored, on return
 *                   undefined; must not overlap any other argument (FBOB_ERR_ALIAS).
 *                   Calls sharing one workspace must be ordered (same stream).
 * Other arguments, outputs and errors as fbob_forward.
 */
int fbob_forward_ws(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                    float tau, int causal,
                    const void* Q, const void* K, const void* V, const void* dO,
                    float* O, float* L, float* D,
                    void* workspace, int64_t workspace_bytes, void* stream);

/*
 * First-order attention backward (FlashAttention blog, "FlashAttention 的反向传播
 * 设计", section 一 for dV = P^T dO, dS = P o (dP - D), dQ = tau dS K,
 * dK = tau dS^T Q, and section 二 for rebuilding P on chip from L).  Two passes
 * like the BoB (FlashBoB notes, "关键设计" 2): a row pass writes dQ and D, then a
 * column pass writes dK and dV (query heads of a group summed on chip); every
 * output is written once, no atomics.
 *
 *   in : Q, dO [B,Hq,N,d], K, V [B,Hkv,N,d] (dtype);
 *        O [B,Hq,N,d], L [B,Hq,N] (fp32) from fbob_forward on the same
 *        (Q, K, V, tau, causal); anything else gives undefined (but
 *        memory-safe) results.
 *   out: dQ [B,Hq,N,d]; dK, dV [B,Hkv,N,d]; D [B,Hq,N] = dO_i . O_i  (fp32).
 *        (O, L, D) is then the complete row state that fbob_bob takes.
 */
int fbob_backward(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                  float tau, int causal,
                  const void* Q, const void* K, const void* V, const void* dO,
                  const float* O, const float* L,
                  float* dQ, float* dK, float* dV, float* D, void* stream);

/*
 * Device workspace, in bytes, that fbob_backward_ws can use for this problem (0 when the
 * problem fills the GPU without splitting: then fbob_backward_ws is fbob_backward).  Same
 * size arguments as fbob_backward; writes the size to *bytes.  FBOB_ERR_INVALID_ARG if
 * bytes is NULL; size errors as fbob_backward.  No HIP call.
 */
int fbob_backward_workspace_size(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                                 int64_t d, float tau, int causal, int64_t* bytes);

/*
 * fbob_backward with a caller-owned device workspace for problems too small to fill the
 * GPU (the same split schedule as fbob_bob_ws, FlashBoB notes, "关键设计" 2): a row-pass
 * work-group owns 256 query rows and a column-pass work-group 256 keys (d = 64) or 128
 * (d = 128); when a pass has too few of them for the 256 CUs, each one's key sweep or
 * row sweep is split over 2-8 work-groups that write fp32 partial sums to the workspace,
 * and a reduction adds them in a fixed order (deterministic; the results differ from
 * fbob_backward's only by the order of the fp32 additions) and writes every output once.
 * bf16 inputs; with causal != 0 or at d = 128 a pass splits only while its tiles do not
 * fill one round of the CUs (unequal tiles dispatched longest first already balance, and
 * at d = 128 splits past one round measured slower).
 *   workspace       DEVICE pointer, 16-byte aligned, owned by the caller, at least
 *                   fbob_backward_workspace_size() bytes; NULL (or fewer bytes) runs
 *                   exactly fbob_backward.  Contents on entry ignored, on return
 *                   undefined; must not overlap any other argument (FBOB_ERR_ALIAS).
 *                   Calls sharing one workspace must be ordered (same stream).
 * Other arguments, outputs and errors as fbob_backward.
 */
int fbob_backward_ws(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                     float tau, int causal,
                     const void* Q, const void* K, const void* V, const void* dO,
                     const float* O, const float* L,
                     float* dQ, float* dK, float* dV, float* D,
                     void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Exact BoB: Pass 1 then Pass 2 on the same stream (FlashBoB notes,
 * "整体框架" flowchart and "关键设计" 2).  No N x N tensor is written to memory;
 * alpha and E are the only state that crosses from Pass 1 to Pass 2.
 *
 *   in : Q, K, V, dO, U_Q [B,Hq,N,d], U_K, U_V [B,Hkv,N,d] (dtype)
 *        O, L, D from fbob_forward on the same (Q, K, V, dO, tau, causal);
 *        anything else gives undefined (but memory-safe) results.
 *   out: dQt, ddOt [B,Hq,N,d]; dKt, dVt [B,Hkv,N,d]; alpha, E [B,Hq,N]  (fp32)
 */
int fbob_bob(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
             float tau, int causal,
             const void* Q, const void* K, const void* V, const void* dO,
             const void* UQ, const void* UK, const void* UV,
             const float* O, const float* L, const float* D,
             float* dQt, float* dKt, float* dVt, float* ddOt,
             float* alpha, float* E, void* stream);

/*
 * Pass 1 alone (row-resident; FlashBoB notes, "关键设计" 2, first pass): streams
 * K, V, U_K, U_V column tiles past a resident row block, accumulates alpha and the
 * five alpha-free accumulators, applies the affine correction of "关键设计" 1
 *   E = E' - alpha D,  ddO~ = ddO~' - alpha o,  dQ~ = tau (Omega - alpha R - E B)
 * and writes dQt, ddOt, alpha, E once.  Same arguments as fbob_bob minus dKt, dVt.
 */
int fbob_bob_pass1(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                   float tau, int causal,
                   const void* Q, const void* K, const void* V, const void* dO,
                   const void* UQ, const void* UK, const void* UV,
                   const float* O, const float* L, const float* D,
                   float* dQt, float* ddOt, float* alpha, float* E, void* stream);

/*
 * Pass 2 alone (column-resident; FlashBoB notes, "关键设计" 2, second pass and
 * "关键设计" 3 for the grouped heads): streams row tiles of Q, dO, U_Q, L, D and
 * the Pass 1 scalars (alpha, E) past a resident K/V column block, and writes
 * dKt, dVt exactly once (the query heads of a group are summed on chip).
 *   in : as fbob_bob, plus alpha, E from fbob_bob_pass1 on the same inputs.
 *   out: dKt, dVt [B,Hkv,N,d] (fp32)
 */
int fbob_bob_pass2(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                   float tau, int causal,
                   const void* Q, const void* K, const void* V, const void* dO,
                   const void* UQ, const void* UK, const void* UV,
                   const float* L, const float* D, const float* alpha, const float* E,
                   float* dKt, float* dVt, void* stream);

/*
 * Device workspace, in bytes, that fbob_bob_ws can use for this problem (0 when the
 * problem fills the GPU without splitting: then fbob_bob_ws is fbob_bob).  Same size
 * arguments as fbob_bob; writes the size to *bytes.  FBOB_ERR_INVALID_ARG if bytes is
 * NULL; size errors as fbob_bob.  No HIP call.
 */
int fbob_bob_workspace_size(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                            float tau, int causal, int64_t* bytes);

/*
 * fbob_bob with a caller-owned device workspace for problems too small to fill the
 * GPU (FlashBoB notes, "关键设计" 2: the same two passes).  A Pass 1 work-group owns
 * 128 query rows and a Pass 2 work-group 256 keys (d = 64) or 128 (d = 128); when a
 * problem has too few tiles to keep the 256 CUs busy (e.g. B=1 H=12 N=4096 d=64),
 * each row tile's key sweep, or each column tile's row sweep, is split over 2-8
 * work-groups that write fp32 partial sums to the workspace, and a reduction kernel
 * adds them in a fixed order (results are deterministic; they differ from
 * fbob_bob's only by the order of the fp32 additions) and writes every output once.
 * When a pass's work-groups fill at least one whole round of the CUs, the heads of the
 * whole rounds run unsplit and only the remaining heads split (where the boundary falls
 * between groups of query heads of one batch, or between batches).
 * Splitting applies to bf16 inputs, d = 64 with tau a power of two or d = 128.  With
 * causal != 0 at d = 64 a work-group of either pass owns two tiles (p and n - 1 - p,
 * so that every work-group has the same masked work) and the split cuts the two
 * tiles' joint sweep into equal parts; at d = 128 each tile's own sweep is cut.
 *   workspace       DEVICE pointer, 16-byte aligned, owned by the caller, at least
 *                   fbob_bob_workspace_size() bytes; NULL (or fewer bytes) runs the
 *                   unsplit schedule, i.e. exactly fbob_bob.  Its contents on entry
 *                   are ignored and on return are undefined; it must not overlap any
 *                   other argument (FBOB_ERR_ALIAS).  Calls sharing one workspace
 *                   must be ordered (same stream), or they race.
 * Other arguments, outputs and errors as fbob_bob.
 */
int fbob_bob_ws(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                float tau, int causal,
                const void* Q, const void* K, const void* V, const void* dO,
                const void* UQ, const void* UK, const void* UV,
                const float* O, const float* L, const float* D,
                float* dQt, float* dKt, float* dVt, float* ddOt,
                float* alpha, float* E, void* workspace, int64_t workspace_bytes,
                void* stream);

/*
 * fbob_bob_ws without a caller-provided workspace and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  When the problem's split
 * schedule needs a workspace (fbob_bob_workspace_size > 0) its partial sums go to a
 * static device array of FBOB_SCRATCH_BYTES (128 MiB) that the library holds on each
 * device it runs on until the process ends; the library allocates nothing and
 * issues no memset (every partial a call reads is written earlier in that call).
 *   * FBOB_ERR_SCRATCH, before any HIP call, if the workspace size exceeds
 *     FBOB_SCRATCH_BYTES (e.g. B=2 H=10 N=4096 d=128 needs 160 MiB); fbob_bob or
 *     fbob_bob_ws serve such problems.
 *   * All calls on one device share that device's array: calls that overlap in
 *     time on one device (on different streams, or from threads without an order
 *     between them) race and give wrong results.  Calls on one stream are ordered.
 *   * `stream` must belong to the current device (FBOB_ERR_INVALID_ARG otherwise);
 *     the array's device address is looked up once per device, on the first call
 *     there that splits.
 * Arguments, outputs and the other errors as fbob_bob; the results are those of
 * fbob_bob_ws with a large enough workspace, bitwise.
 */
int fbob_bob_noalloc(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                     float tau, int causal,
                     const void* Q, const void* K, const void* V, const void* dO,
                     const void* UQ, const void* UK, const void* UV,
                     const float* O, const float* L, const float* D,
                     float* dQt, float* dKt, float* dVt, float* ddOt,
                     float* alpha, float* E, void* stream);

/* Bits of fbob_bob_ex's flags argument. */
#define FBOB_FLAG_FP32_ROW_SUMS 1

/*
 * fbob_bob_ws with options: `flags` is a bitwise OR of FBOB_FLAG_* values, and
 * flags = 0 gives fbob_bob_ws's results bitwise.
 *   FBOB_FLAG_FP32_ROW_SUMS  (bf16 inputs, d = 64) Pass 1 forms the row sums
 *     alpha_i = sum_j P_ij F_ij and E'_i = sum_j P_ij dP~'_ij (FlashBoB notes,
 *     "关键设计" 1, the alpha-free accumulators) as fp32 sums of the unrounded
 *     products.  Without it alpha is summed from the same bf16-rounded P F that
 *     feed the ddO~ contraction, and E' is taken as dO_i . ddO~_i: the rounding then
 *     cancels in ddO~ = ddO~' - alpha o but stays in alpha (relative ~2^-9 of
 *     sum_j |P_ij F_ij|), and every dK~ and dV~ column takes alpha_i and E_i of each
 *     row.  With the flag alpha and E carry fp32 rounding only, so dK~ and dV~ improve
 *     where rows are near one-hot with large F; ddO~ no longer cancels the rounding
 *     of P F and its error grows by a small factor.  Pass 1 takes a few percent
 *     longer.  With f32 inputs no product is rounded to bf16, and at d = 128 the row
 *     sums are always fp32 lane sums: there the flag changes nothing.
 *   Any other bit: FBOB_ERR_INVALID_ARG, before any HIP call.
 * Workspace, the other arguments, outputs and errors as fbob_bob_ws.
 */
int fbob_bob_ex(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                float tau, int causal, int flags,
                const void* Q, const void* K, const void* V, const void* dO,
                const void* UQ, const void* UK, const void* UV,
                const float* O, const float* L, const float* D,
                float* dQt, float* dKt, float* dVt, float* ddOt,
                float* alpha, float* E, void* workspace, int64_t workspace_bytes,
                void* stream);

/*
 * Name of the HIP error behind the calling thread's last FBOB_ERR_HIP (a static string,
 * e.g. "hipErrorInvalidConfiguration"), or "no HIP error" if that thread has had none.
 * Thread-local; no GPU call.
 */
const char* fbob_hip_error_string(void);

/* Static string naming a status code ("unknown status" for other values). */
const char* fbob_strerror(int status);

/* FBOB_VERSION of the built library. */
int fbob_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FBOB_H_ */

/*
 * ckda.h -- C ABI of the MI355X (gfx950) CKDA / KDA kernel library.
 *
 * The library computes the (Complex) Kimi Delta Attention recurrence, one
 * independent state per (batch, head):
 *
 *   H_t = (I - beta_t k_t k_t^T) Diag(alpha_t) H_{t-1} + beta_t k_t v_t^T
 *   o_t = H_t^T q_t
 *
 * with H_t of shape d_k x d_v (row i = key channel i) and unit-norm keys
 * ("Complex KDA", Eq. (1); discussion slides, frame "CKDA keeps the original
 * gate--delta--readout structure").  KDA ranges (alpha in (0,1], beta in
 * [0,1]) and CKDA ranges (alpha in [-1,1], beta in [0,2], Sec. 3 "CKDA")
 * run through the same code: signed gates are split into a sign and a
 * magnitude and the cumulative signs are absorbed into keys and queries
 * inside the kernels (discussion slides, frame "Absorb cumulative signs into
 * keys and queries"; paper Prop. 2 for sign(0) = +1).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers owned by the caller.  The library allocates
 *   no device memory and keeps no state between calls apart from a
 *   thread-local error string.
 * - Tensors are contiguous, C order, base addresses 16-byte aligned.
 * - `dtype` (ckda_dtype_t) is the element type of q, k, v, alpha, beta and o.
 *   States (h0, hT, H_inout) are always fp32.
 * - q is not scaled and k is not normalised: the caller supplies ||k_t|| = 1
 *   (the *_ex entry points can normalise both and form the gates from
 *   logits, see CKDA_FUSE_*).  alpha and beta are used as given (no clamping
 *   of range violations).  The one exception is internal to the chunked
 *   forward's intra-chunk Gram matrices, where a gate magnitude below 2^-31
 *   counts as 2^-31 (sign kept): that changes a decay only where its exact
 *   value is below 2^-31 already; see ckda_chunk_fwd.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *   and the call returns without waiting.  The return value reports argument
 *   errors (detected before anything is launched) and launch errors; faults
 *   during execution surface at the caller's next synchronisation.
 * - Errors: every function returns a ckda_status_t; nothing aborts or throws
 *   across the ABI.  ckda_last_error() returns a thread-local description of
 *   the last non-OK status.
 * - Results are bitwise deterministic run to run (no atomics, fixed
 *   reduction order).  Calls on different streams with disjoint buffers may
 *   run concurrently.
 */
#ifndef CKDA_H
#define CKDA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CKDA_ABI_VERSION 1

typedef enum { CKDA_DTYPE_F32 = 0, CKDA_DTYPE_BF16 = 1 } ckda_dtype_t;

/* Codes 0-5 are the boundary's original set; codes added later follow them. */
typedef enum {
  CKDA_OK = 0,
  CKDA_ERR_NULL = 1,        /* a required pointer is NULL */
  CKDA_ERR_DIM = 2,         /* a size is negative or inconsistent */
  CKDA_ERR_UNSUPPORTED = 3, /* valid but not supported (dtype, d_k, d_v, chunk) */
  CKDA_ERR_ALIAS = 4,       /* an output overlaps an input it may not overlap */
  CKDA_ERR_HIP = 5,         /* the HIP runtime reported an error at launch */
  CKDA_ERR_WORKSPACE = 6,   /* workspace missing, too small or misaligned */
  CKDA_ERR_FLAGS = 7        /* flags hold bits outside CKDA_FUSE_* / CKDA_GATE_SCALAR */
} ckda_status_t;

/* Per-token prologue steps of the *_ex entry points (bitwise OR; 0 = none,
 * the inputs are used as given, exactly as by the plain entry points).  They
 * follow the practical parameterisation of the "Complex KDA" discussion
 * slides (frame "Backup: practical gates differ from exact theoretical
 * endpoints") and the unit-norm keys the recurrence assumes (frame "Absorb
 * cumulative signs into keys and queries"), and are computed in fp32 inside
 * the kernels, with no extra pass over memory:
 *
 *   CKDA_FUSE_GATES   alpha and beta hold logits a, b:
 *                       alpha = s (eps + (1 - eps) |tanh(a / 2)|),  eps = e^-5,
 *                       s = +1 for a >= 0 (a = -0 included), else -1,
 *                       beta  = 2 sigmoid(b),
 *                     so |alpha| in [e^-5, 1] (fp32), sign free, beta in [0, 2].
 *   CKDA_FUSE_NORM_K  each key row is scaled to unit norm: k / sqrt(|k|^2 + 1e-6)
 *                     (the guard, which the pages do not give, maps a zero key
 *                     to zero and moves a unit key by 5e-7).
 *   CKDA_FUSE_NORM_Q  the same for each query row.
 *
 * In the chunked forward with CKDA_FUSE_GATES the computed gates stay fp32
 * (they are not rounded to dtype) before they enter the chunk products. */
#define CKDA_FUSE_GATES 1
#define CKDA_FUSE_NORM_K 2
#define CKDA_FUSE_NORM_Q 4

/* Gate shape flag of ckda_chunk_fwd_ex and ckda_decode_step_ex: alpha holds
 * ONE gate per token and head ([B, H, T] / [N, H]) applied to every key
 * channel -- the scalar gate of Gated DeltaNet, a comparator of the "Complex
 * KDA" paper (Sec. 2, scalar gates commute with every matrix and leave the
 * transition symmetric).  Combines with CKDA_FUSE_GATES (the scalar is then a
 * logit) and the norm flags; not with a channel gather. */
#define CKDA_GATE_SCALAR 8

/* Bytes of device workspace ckda_chunk_fwd needs for these sizes, or 0 when
 * the sizes are invalid or unsupported (ckda_chunk_fwd then reports why).
 * The workspace holds, per chunk of every (batch, head), the operands the
 * state pass consumes (see ckda_chunk_fwd): the blocks on or below the
 * diagonal of two chunk x chunk lower-triangular matrices (for bf16 one of
 * them twice, as a hi and a lo part), 3*chunk*d_k elements of dtype and d_k
 * floats, in whole 1 KB blocks (bf16, chunk 64, d_k 128: 67 KB per chunk). */
size_t ckda_chunk_fwd_workspace_size(int B, int H, int T, int dk, int dv, int chunk, int dtype);

/* Chunkwise-parallel forward over a whole sequence for every (batch, head).
 *
 *   q, k, alpha : [B, H, T, dk]  dtype
 *   v           : [B, H, T, dv]  dtype
 *   beta        : [B, H, T]      dtype
 *   h0          : [B, H, dk, dv] fp32 initial states, or NULL for zeros
 *   o           : [B, H, T, dv]  dtype, o_t = H_t^T q_t (post-update state)
 *   hT          : [B, H, dk, dv] fp32 final states, or NULL to skip
 *   workspace   : device buffer of at least ckda_chunk_fwd_workspace_size()
 *                 bytes, 256-byte aligned; contents on entry are ignored and
 *                 on return are unspecified.  It must not overlap any other
 *                 argument.
 *
 * Supported: dtype F32 or BF16; dk, dv in {16, 32, 64, 128}; chunk in
 * {16, 32, 64}; any T >= 0 (T = 0 copies h0 to hT, or zeros).  A last chunk
 * shorter than `chunk` is handled exactly (the missing positions act as
 * identity steps and are not stored).
 *
 * Aliasing: o must not overlap any input; hT may equal h0 exactly (in-place
 * continuation of a state) but must not otherwise overlap an input.
 *
 * The result equals the sequential recurrence up to floating-point rounding
 * (the KDA course lesson, "Chunkwise execution": chunking changes cost, not
 * the numbers), computed in two kernels.  A Gram kernel, parallel over all
 * chunks, forms each chunk's signed gate products, its decayed Gram matrices
 * and the unit lower-triangular (UT/WY) solve, and writes the chunk's state-
 * independent operands to the workspace.  A state-pass kernel carries the
 * fp32 state from chunk to chunk and emits the outputs.  bf16 inputs are
 * multiplied on bf16 matrix cores with fp32 accumulation (the state's chain
 * from chunk to chunk with split hi + lo bf16 operands); fp32 inputs on fp32
 * matrix cores.  The workspace argument is this entry point's one departure
 * from a plain (inputs, outputs, sizes, stream) call: the two kernels hand
 * the per-chunk operands over through it, and the library allocates nothing
 * (ckda_chunk_fwd_noalloc takes the plain signature and a fixed buffer).
 *
 * Gate range: the paper's CKDA range is |alpha| <= 1 (App. B.2).  Gates of
 * larger modulus are computed as given (no clamp, no error); the chunk
 * kernels rescale by products of a chunk's gates, so results stay accurate
 * while those products stay far from the fp32 limits (tested with |alpha| up
 * to 1.25).  Gate magnitudes below 2^-31 enter the Gram factors as 2^-31
 * (sign kept); the products that reach the outputs use the gates as given. */
int ckda_chunk_fwd(const void* q, const void* k, const void* v, const void* alpha,
                   const void* beta, const float* h0, void* o, float* hT,
                   int B, int H, int T, int dk, int dv, int chunk, int dtype,
                   void* workspace, size_t workspace_bytes, void* stream);

/* ckda_chunk_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without the workspace, the same checks and results.
 * The chunk records live in the library's one fixed device buffer, 64 MiB
 * per GPU, held from the first call on that GPU until the process ends; the
 * call itself allocates nothing.  Heads run in batches that fill the buffer
 * (one Gram and one state-pass launch per batch, in order on `stream`).
 *
 * Limit: one head's records (ckda_chunk_fwd_workspace_size(1, 1, T, dk, dv,
 * chunk, dtype) bytes; bf16, chunk 64, d_k 128: about 1.05 KB per position,
 * T <= 62,000) must fit the buffer, else CKDA_ERR_WORKSPACE.
 *
 * All calls on one GPU share its buffer: calls that overlap in time on one
 * GPU (different streams, or different host threads) race and corrupt each
 * other's results; calls on one stream are ordered and safe.  Errors as
 * ckda_chunk_fwd (CKDA_ERR_HIP if the buffer's address cannot be found). */
int ckda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* alpha,
                           const void* beta, const float* h0, void* o, float* hT,
                           int B, int H, int T, int dk, int dv, int chunk, int dtype, void* stream);

/* ckda_chunk_fwd with timing marks, for measurement: identical arguments,
 * checks and results, and in addition each non-NULL event (a hipEvent_t the
 * caller created on the current device) is recorded on `stream` -- ev_start
 * before the Gram kernel, ev_mid between the Gram and the state-pass kernel,
 * ev_end after the state-pass kernel -- so that the caller can read each
 * kernel's duration with hipEventElapsedTime after synchronising.  The events
 * stay owned by the caller. */
int ckda_chunk_fwd_timed(const void* q, const void* k, const void* v, const void* alpha,
                         const void* beta, const float* h0, void* o, float* hT,
                         int B, int H, int T, int dk, int dv, int chunk, int dtype,
                         void* workspace, size_t workspace_bytes, void* stream,
                         void* ev_start, void* ev_mid, void* ev_end);

/* ckda_chunk_fwd with the per-token prologue `flags` (CKDA_FUSE_*) applied
 * to the inputs first: alpha and beta may be logits, k and q are normalised
 * per token.  The prologue's results are not written anywhere.  Same
 * arguments, layouts, aliasing rules and workspace as ckda_chunk_fwd; flags
 * = 0 gives ckda_chunk_fwd's results exactly.  With CKDA_GATE_SCALAR alpha
 * is [B, H, T].  Returns CKDA_ERR_FLAGS for unknown bits. */
int ckda_chunk_fwd_ex(const void* q, const void* k, const void* v, const void* alpha,
                      const void* beta, const float* h0, void* o, float* hT,
                      int B, int H, int T, int dk, int dv, int chunk, int dtype, int flags,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ckda_chunk_fwd_ex on a retained subset of key channels, gathered inside
 * the kernels (the state-reduction setting of the "On State Reduction in
 * Linear Attention" presentation: a per-head index set keeps dk of the dk_in
 * key/query channels, and the recurrence runs on the kept ones).
 *
 *   q, k, alpha : [B, H, T, dk_in] dtype, full-width rows
 *   idx         : [H, dk] int32 DEVICE array; head h uses channels
 *                 idx[h][0..dk-1] of its rows, in that order (repeats
 *                 allowed).  An index outside [0, dk_in) is clamped into it
 *                 (no fault; the result is then unspecified).
 *   v, beta, h0, o, hT, workspace : as ckda_chunk_fwd, with dk the KEPT width
 *                 (states [B, H, dk, dv]; workspace size for dk).
 *
 * Equivalent to ckda_chunk_fwd_ex on q, k, alpha gathered beforehand
 * (x[..., idx[h]]) without that extra pass over memory; with CKDA_FUSE_NORM_K
 * the keys are normalised over the kept channels.  1 <= dk_in <= 65536; idx
 * must be 16-byte aligned and must not overlap an output. */
int ckda_chunk_fwd_gather(const void* q, const void* k, const void* v, const void* alpha,
                          const void* beta, const float* h0, void* o, float* hT,
                          int B, int H, int T, int dk_in, const int* idx, int dk, int dv, int chunk, int dtype,
                          int flags, void* workspace, size_t workspace_bytes, void* stream);

/* DeltaProduct_2 forward: two delta-rule sub-steps per token, each with its
 * own key, value and beta, and one read-out per token after both (the
 * DeltaProduct_2 comparator of the "Complex KDA" paper, Fig. 5 and Sec. 6,
 * where it runs ungated; App. C's Gated DeltaProduct scales the product of
 * the sub-steps' Householder factors by one scalar gate per token):
 *
 *   Hb = alpha_t H_{t-1}            (alpha_t = 1 when alpha is NULL)
 *   H' = Hb + beta_t1 k_t1 (v_t1 - Hb^T k_t1)^T
 *   H_t = H' + beta_t2 k_t2 (v_t2 - H'^T k_t2)^T,   o_t = H_t^T q_t
 *
 *   q           : [B, H, T, dk]      dtype
 *   k           : [B, H, T, 2, dk]   dtype (sub-step keys k_t1, k_t2)
 *   v           : [B, H, T, 2, dv]   dtype
 *   beta        : [B, H, T, 2]       dtype
 *   alpha       : [B, H, T] dtype scalar gates, or NULL (ungated)
 *   h0, hT      : [B, H, dk, dv] fp32 as ckda_chunk_fwd;  o : [B, H, T, dv]
 *   workspace   : ckda_chunk_fwd_workspace_size(B, H, 2 * T, dk, dv, chunk, dtype) bytes
 *
 * The 2 T sub-steps run through the chunked forward's kernels as one
 * sequence (k, v and beta above are that sequence in memory order); only the
 * second sub-step of each token is read out.  flags: CKDA_FUSE_* (the norm
 * flags normalise every sub-step key and the query; CKDA_FUSE_GATES makes
 * beta, and alpha if given, logits).  Other rules as ckda_chunk_fwd. */
int ckda_deltaproduct2_fwd(const void* q, const void* k, const void* v, const void* alpha,
                           const void* beta, const float* h0, void* o, float* hT,
                           int B, int H, int T, int dk, int dv, int chunk, int dtype, int flags,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace ckda_chunk_bwd needs, or 0 for invalid or
 * unsupported sizes: per 32-position chunk of every (batch, head) an fp32
 * record (5 * 32 * 32 + 5 * 32 * dk + dk floats, rounded up to 64 floats)
 * plus the chunk-start state and its gradient (2 * dk * dv floats). */
size_t ckda_chunk_bwd_workspace_size(int B, int H, int T, int dk, int dv, int dtype);

/* Backward of the chunked forward: the gradients of a loss L with respect to
 * every input, given do = dL/do and dhT = dL/dH_T.
 *
 *   q, k, v, alpha, beta, h0 : the forward's inputs (layouts, dtype and h0 as
 *                 ckda_chunk_fwd; h0 NULL = zero initial state)
 *   dout        : [B, H, T, dv] dtype, dL/do
 *   dhT         : [B, H, dk, dv] fp32 dL/dH_T, or NULL for zero
 *   dq, dk, dalpha : [B, H, T, dk] fp32;  dv : [B, H, T, dv] fp32
 *   dbeta       : [B, H, T] fp32;  dh0 : [B, H, dk, dv] fp32, or NULL to skip
 *   workspace   : at least ckda_chunk_bwd_workspace_size() bytes, 256-byte
 *                 aligned, contents ignored on entry and unspecified on return
 *
 * The reverse-mode derivative of the recurrence of ckda_chunk_fwd (paper
 * Eq. (1)) with the gates as the signed numbers they are: dalpha is the plain
 * partial derivative, exact at zero gates, and no gate is floored or divided
 * by (a gate derivative collects every pair of positions across it with the
 * gate's own factor left out).  Computed in fp32 from the inputs (the forward's
 * workspace is not needed): a chunk-parallel pass forms each 32-position
 * chunk's solve and decayed Gram matrices, two sequential passes carry the
 * state forward and its gradient backward from chunk to chunk, and a
 * chunk-parallel pass forms every per-token gradient.  The CKDA_FUSE_*
 * prologue is not differentiated here (the gradients are with respect to the
 * gates, beta and vectors the recurrence consumes).
 *
 * Supported: dtype F32 or BF16; dk, dv in {16, 32, 64, 128}; any T >= 0.
 * Outputs must not overlap each other, any input or the workspace. */
int ckda_chunk_bwd(const void* q, const void* k, const void* v, const void* alpha, const void* beta,
                   const float* h0, const void* dout, const float* dhT, float* dq, float* dk, float* dv,
                   float* dalpha, float* dbeta, float* dh0, int B, int H, int T, int dk_, int dv_, int dtype,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace ckda_chunk_bwd_ex needs for these sizes and
 * flags, or 0 when they are invalid or unsupported.  With flags 0 it equals
 * ckda_chunk_bwd_workspace_size; otherwise it also holds the prologue's
 * outputs, v and do in fp32 (3 dk + 2 dv + 1 floats per token and head, plus
 * dk more with CKDA_GATE_SCALAR). */
size_t ckda_chunk_bwd_ex_workspace_size(int B, int H, int T, int dk, int dv, int dtype, int flags);

/* Backward of ckda_chunk_fwd_ex: the gradients with respect to the raw
 * inputs the fused forward takes.  `flags` as ckda_chunk_fwd_ex
 * (CKDA_FUSE_GATES, CKDA_FUSE_NORM_K, CKDA_FUSE_NORM_Q, CKDA_GATE_SCALAR):
 *   CKDA_FUSE_GATES  dalpha, dbeta are the gradients with respect to the
 *                    logits a, b.  The gate's backward follows the "Complex
 *                    KDA" discussion slides (frame "Backup: practical gates
 *                    differ from exact theoretical endpoints"): the sign s is
 *                    held constant and |tanh(a/2)| takes the zero subgradient
 *                    at 0, so d alpha/d a = (1 - e^-5)(1 - tanh(a/2)^2)/2 for
 *                    a != 0 and 0 at a = 0 (the jump of the gate at 0 passes
 *                    no gradient); d beta/d b = 2 sigma(b)(1 - sigma(b)).
 *   CKDA_FUSE_NORM_K / _NORM_Q  dk / dq are with respect to the raw rows:
 *                    dx = n (dy - y (y . dy)), y = x n, n = (|x|^2 + 1e-6)^-1/2.
 *   CKDA_GATE_SCALAR alpha (and dalpha) are [B, H, T]: one gate per token and
 *                    head; its gradient sums those of the channels it gates.
 * Other arguments, layouts and rules as ckda_chunk_bwd (dv and dh0 are
 * unaffected by the prologue).  With flags 0 this is ckda_chunk_bwd.
 * Otherwise the prologue's outputs (and v, do) are first written to the
 * workspace in fp32, the fp32 backward runs on them, and a last pass maps the
 * gradients back through the prologue, one token row per wave.
 * Errors: CKDA_ERR_FLAGS for unknown flag bits; others as ckda_chunk_bwd. */
int ckda_chunk_bwd_ex(const void* q, const void* k, const void* v, const void* alpha, const void* beta,
                      const float* h0, const void* dout, const float* dhT, float* dq, float* dk, float* dv,
                      float* dalpha, float* dbeta, float* dh0, int B, int H, int T, int dk_, int dv_, int dtype,
                      int flags, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace ckda_deltaproduct2_bwd needs, or 0 when the
 * sizes are invalid or unsupported: the sub-step queries, gates and upstream
 * gradients (2 T rows, dtype), two fp32 sub-step gradient arrays and the
 * chunked backward's workspace for 2 T steps. */
size_t ckda_deltaproduct2_bwd_workspace_size(int B, int H, int T, int dk, int dv, int dtype);

/* Backward of ckda_deltaproduct2_fwd ("Complex KDA" paper, Fig. 5 and
 * Sec. 6; gated form App. C): the gradients of a loss with respect to every
 * input, given do = dL/do [B, H, T, dv] (dtype) and dhT = dL/dH_T (fp32 or
 * NULL).  Layouts as the forward: k, dk [B, H, T, 2, dk]; v, dv
 * [B, H, T, 2, dv]; beta, dbeta [B, H, T, 2]; q, dq [B, H, T, dk]; alpha and
 * dalpha [B, H, T] (alpha NULL: ungated, dalpha ignored); gradients fp32.
 * DeltaProduct_2 is the delta rule over the 2 T sub-steps (the gate on the
 * first of each token's two, the query read after the second), so this runs
 * the chunked backward of ckda_chunk_bwd on that sequence and folds each
 * token's two sub-step query gradients and its gate sub-step's channel
 * gradients.  Errors and rules as ckda_chunk_bwd. */
int ckda_deltaproduct2_bwd(const void* q, const void* k, const void* v, const void* alpha, const void* beta,
                           const float* h0, const void* dout, const float* dhT, float* dq, float* dk, float* dv,
                           float* dalpha, float* dbeta, float* dh0, int B, int H, int T, int dk_, int dv_, int dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

/* One recurrent decode step for N sequences x H heads, state in place.
 *
 *   q, k, alpha : [N, H, dk]     dtype
 *   v           : [N, H, dv]     dtype
 *   beta        : [N, H]         dtype
 *   H_inout     : [N, H, dk, dv] fp32, read and overwritten with H_t
 *   o           : [N, H, dv]     dtype, o = H_t^T q
 *
 * Computes, per state, in a single read and a single write of H:
 *   s = H^T (alpha . k),  r = H^T (alpha . q),  u = beta (v - s),
 *   o = r + (k^T q) u,    H <- Diag(alpha) H + k u^T
 * which is the read-compare-correct step of the KDA course lesson
 * ("Mechanism map": S' = diag(a) S, S = S' + beta k (v - S'^T k)^T) read out
 * after the update; the state's diagonal-plus-rank-one structure keeps the
 * work at O(dk dv) per token (discussion slides, "The transition remains
 * non-expansive and inexpensive").  All arithmetic is fp32; no gate floor.
 *
 * Supported: dtype F32 or BF16; dk, dv in {16, 32, 64, 128}; N, H >= 0.
 * Aliasing: o must not overlap H_inout or any input; H_inout must not overlap
 * any input. */
int ckda_decode_step(const void* q, const void* k, const void* v, const void* alpha,
                     const void* beta, float* H_inout, void* o,
                     int N, int H, int dk, int dv, int dtype, void* stream);

/* ckda_decode_step with the per-token prologue `flags` (CKDA_FUSE_*) applied
 * to the token first (fp32 throughout).  Same arguments and rules as
 * ckda_decode_step; flags = 0 gives its results exactly.  With
 * CKDA_GATE_SCALAR alpha is [N, H].  Returns CKDA_ERR_FLAGS for unknown bits. */
int ckda_decode_step_ex(const void* q, const void* k, const void* v, const void* alpha,
                        const void* beta, float* H_inout, void* o,
                        int N, int H, int dk, int dv, int dtype, int flags, void* stream);

/* One DeltaProduct_2 decode step (the recurrence of ckda_deltaproduct2_fwd)
 * for N sequences x H heads, state in place, in one read and one write of
 * the state:  q [N, H, dk], k [N, H, 2, dk], v [N, H, 2, dv], beta [N, H, 2],
 * alpha [N, H] scalar gates or NULL, H_inout [N, H, dk, dv] fp32, o [N, H, dv].
 * flags: CKDA_FUSE_*.  All arithmetic fp32. */
int ckda_deltaproduct2_decode_step(const void* q, const void* k, const void* v, const void* alpha,
                                   const void* beta, float* H_inout, void* o,
                                   int N, int H, int dk, int dv, int dtype, int flags, void* stream);

/* ckda_decode_step_ex on a retained subset of key channels gathered inside
 * the kernel: q, k, alpha are [N, H, dk_in] full-width rows, idx [H, dk]
 * int32 device indices (as ckda_chunk_fwd_gather), the state [N, H, dk, dv]
 * covers the kept channels. */
int ckda_decode_step_gather(const void* q, const void* k, const void* v, const void* alpha,
                            const void* beta, float* H_inout, void* o,
                            int N, int H, int dk_in, const int* idx, int dk, int dv, int dtype, int flags,
                            void* stream);

/* Static description of a status code. */
const char* ckda_status_string(int status);

/* Thread-local detail of the last non-OK status returned on this thread
 * (empty string if none).  Valid until the next call on this thread. */
const char* ckda_last_error(void);

/* CKDA_ABI_VERSION of the built library. */
int ckda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CKDA_H */

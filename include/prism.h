/*
 * prism.h -- C ABI of the PRISM layer hot path on AMD MI355X (gfx950).
 *
 * The layer is the one described by the web summary "Technical Summary: PRISM
 * (Parallel Residual Iterative Sequence Model)" (gist.science, paper
 * 2602.10796), sections cited as §n below:
 *
 *   Stage 1 (§2.2): u_t = sum_{j=0..3} conv[h, :, j] * v_{t-j}      (ShortConv anchor)
 *   Stage 2 (§2.2): r^(1) = v_t - u_t; for l = 1..L:
 *                   k^(l) = W_k^(l) u_t, p^(l) = W_p^(l) u_t,
 *                   beta^(l) = sigmoid(w_beta^(l) . u_t),
 *                   delta^(l) = GELU(p^(l) * r^(l)), r^(l+1) = r^(l) - delta^(l)
 *   Write   (§2.2): B_t = beta_t v_t k_t^T + sum_l beta^(l) delta^(l) k^(l)^T
 *   Forget  (§2.1): A_t = alpha_t (I - beta_t k_t k_t^T)   (Gated-DeltaNet form)
 *   Update  (§2.1): S_t = S_{t-1} A_t + B_t
 *   Readout        : o_t = S_t q_t
 * With L = 0 the layer is Gated DeltaNet (§3, item 3).  GELU is the exact erf
 * form.  The base term beta_t v_t k_t^T of the write, r^(1) = v - u, the conv
 * over v of width 4 (tap j multiplies v_{t-j}), the gate beta^(l) as a
 * sigmoid of w_beta^(l) . u and the readout are readings of passages the
 * summary leaves open; the library implements exactly the formulas above.
 *
 * Conventions common to every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers, contiguous, row-major, 16-byte
 *   aligned.  The caller owns every buffer, including the workspace.  The
 *   library allocates no device memory and keeps no pointer after a call.
 * - Work is enqueued asynchronously on `stream`; nothing synchronises the
 *   host.  Buffers must stay alive until the stream has finished the work.
 * - Every argument is validated on the host before any HIP call; a failed
 *   check returns a non-zero status and enqueues nothing.
 *   prism_last_error() then returns a message naming the argument.
 * - NaN / Inf inputs are not checked; they propagate.
 * - Results are deterministic: the same inputs and descriptor give bitwise
 *   identical outputs (no atomics; all reductions in a fixed order).
 * - Functions are thread-safe except while kernel timing is enabled
 *   (prism_timing_begin .. prism_timing_end).
 */
#ifndef PRISM_H_
#define PRISM_H_

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PRISM_OK = 0,
  PRISM_ERR_NULL = 1,        /* a required pointer is NULL                      */
  PRISM_ERR_SHAPE = 2,       /* a size is out of range (B, T, H < 1, ...)       */
  PRISM_ERR_UNSUPPORTED = 3, /* valid but outside the compiled envelope         */
  PRISM_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                */
  PRISM_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required         */
  PRISM_ERR_HIP = 6          /* a HIP launch failed; see prism_last_error()     */
} prism_status;

typedef enum {
  PRISM_F32 = 0,  /* q, k, v, o, weights, taps, dO, dq, dk, dv in float32  */
  PRISM_BF16 = 1  /* the same tensors in bfloat16 (round-to-nearest-even)  */
} prism_dtype;

/* Refinement step activation (summary §2.2 "Residual Update"): the step
 * correction is delta = GELU(p * r) (the method) or delta = p * r (the
 * ablation without the nonlinearity). */
typedef enum {
  PRISM_ACT_GELU = 0,
  PRISM_ACT_IDENTITY = 1
} prism_activation;

/* Problem descriptor.
 *   B, T, H    batch, sequence length, heads            (each >= 1;
 *              H * dk <= 4194304)
 *   dk, dv     key / value head dimension; must be equal, in {16, 32, 64, 128}
 *              for PRISM_BF16 and {16, 32, 64} for PRISM_F32
 *   L          refinement steps, 0 <= L <= 8
 *   chunk      tokens per chunk of the parallel scan, in {16, 32, 64}
 *              (PRISM_F32 also needs dk * chunk <= 2048); any T >= 1 is
 *              accepted (the last chunk may be partial)
 *   conv_width ShortConv width; must be 4
 *   dtype      storage type of the dtype-typed tensors (see prism_dtype)
 *   activation refinement step activation, a prism_activation value
 *              (0 = GELU, the method's step)
 *   conv_offset ShortConv tap offset: 0 = tap j multiplies v_{t-j} (the
 *              current token and the three before it), 1 = tap j multiplies
 *              v_{t-1-j} (strictly past tokens, the ones the state S_{t-1}
 *              has seen; summary §2.2 Stage 1)
 *   packed_tokens  with cu_seqlens (packed batch, below): N, the number of
 *              token rows in the packed tensors; must be >= 0.  Ignored for
 *              a dense batch.
 * A zero-initialised tail (activation = conv_offset = 0) is the method as
 * described.  activation and conv_offset are ignored when L = 0.           */
typedef struct {
  int B, T, H, dk, dv, L, chunk, conv_width;
  prism_dtype dtype;
  int activation, conv_offset;
  int packed_tokens;
} prism_desc;

/* Tensor layouts (element type "dt" = desc->dtype; f32 = float32):
 *   q, k        [B, T, H, dk]  dt      v, o, dO   [B, T, H, dv]  dt
 *   alpha, beta [B, T, H]      f32     alpha in (0, 1], beta in [0, 1]
 *   Wk          [H, L, dk, dv] dt      k^(l) = Wk[h, l] u   (row i . u)
 *   Wp          [H, L, dv, dv] dt      p^(l) = Wp[h, l] u
 *   wbeta       [H, L, dv]     dt      beta^(l) = sigmoid(wbeta[h, l] . u)
 *   conv        [H, dv, 4]     dt      tap j multiplies v_{t-j} (j = 0: current token),
 *                                      or v_{t-1-j} with conv_offset = 1
 *   conv_hist   [B, 4, H, dv]  dt      v_{-4} .. v_{-1}: the four values before the
 *                                      sequence, oldest first (v's own layout)
 *   S0, ST      [B, H, dv, dk] f32     state entering / leaving the sequence
 *   dST, dS0    [B, H, dv, dk] f32
 *   dq, dk, dv  as q, k, v     dt
 *   dalpha, dbeta [B, T, H]    f32
 *   dWk, dWp, dwbeta, dconv    f32, layouts of Wk, Wp, wbeta, conv
 *   dconv_hist  [B, 4, H, dv]  f32
 * q and k are used as given (callers normalise them if they wish).  With
 * L = 0, Wk, Wp, wbeta, conv (and their gradients) may be NULL.
 *
 * Packed batches (variable lengths).  With cu_seqlens (a device array of
 * B + 1 int32 offsets, 4-byte aligned; NULL = dense) the token tensors q, k,
 * v, o, dO, dq, dk, dv are [N, H, d] and alpha, beta, dalpha, dbeta [N, H],
 * N = desc->packed_tokens, sequence b being tokens cu_seqlens[b] ..
 * cu_seqlens[b+1] - 1; desc->T is then the longest length (it sizes the
 * workspaces).  Meant: cu_seqlens[0] = 0, non-decreasing, cu_seqlens[B] = N,
 * every length <= desc->T (lengths of 0 are allowed: S_T = S0).  The offsets
 * are read on the device only: before any kernel uses them, a sanitising
 * pass replaces them by c'_i = max_{j <= i} min(max(cu_seqlens[j], 0), N),
 * and sequences longer than T are cut at T.  Offsets outside the contract
 * therefore give results for those clamped sequences (rows of o and of the
 * gradients outside every clamped sequence are not written), but no access
 * outside the N rows.  conv_hist, S0, ST and their gradients stay per
 * sequence.  A packed batch computes exactly what each sequence would
 * compute alone.
 *
 * Continuation.  A sequence split over several calls gives the same result
 * as one call when each call after the first receives S0 = the previous ST
 * and conv_hist = the previous call's conv_hist_out (summary §2.1: the state
 * carries the past; §2.2 Stage 1: the ShortConv reads the last few values).
 * NULL conv_hist means zeros before the sequence. */

/* Workspace sizes in bytes for a descriptor; *bytes = 0 on error.  The
 * training pair (below) keeps most intermediates in its saved buffer, so its
 * entry points need the (smaller) sizes of the *_train_workspace queries. */
prism_status prism_forward_workspace(const prism_desc* desc, size_t* bytes);
prism_status prism_backward_workspace(const prism_desc* desc, size_t* bytes);
prism_status prism_forward_train_workspace(const prism_desc* desc, size_t* bytes);
prism_status prism_backward_train_workspace(const prism_desc* desc, size_t* bytes);

/* Forward pass: o = readout of S_1..S_T, ST = S_T (ST may be NULL).
 * S0 may be NULL (zero initial state); conv_hist may be NULL (zeros).
 * conv_hist_out (may be NULL) receives the four values of v before the end
 * of the sequence (from conv_hist, or zeros, where T < 4); it may be the same
 * buffer as conv_hist, which is then updated in place after every read. */
prism_status prism_forward(const prism_desc* desc, const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta, const void* Wk, const void* Wp,
                           const void* wbeta, const void* conv, const float* S0,
                           const void* conv_hist, const int* cu_seqlens, void* o, float* ST,
                           void* conv_hist_out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Backward pass: gradients of <dO, o> + <dST, S_T> with respect to every
 * input.  Stateless: recomputes what it needs from the forward inputs.
 * dST may be NULL (zero).  dS0 and dconv_hist may be NULL; each is written
 * when given (dconv_hist is the gradient with respect to conv_hist, zero
 * when L = 0).  Every other gradient pointer is required (weight / tap
 * gradients only when L > 0).  Gradients are written, not accumulated. */
prism_status prism_backward(const prism_desc* desc, const void* q, const void* k, const void* v,
                            const float* alpha, const float* beta, const void* Wk, const void* Wp,
                            const void* wbeta, const void* conv, const float* S0,
                            const void* conv_hist, const int* cu_seqlens, const void* dO,
                            const float* dST, void* dq, void* dk, void* dv, float* dalpha,
                            float* dbeta, float* dWk, float* dWp, float* dwbeta, float* dconv,
                            float* dS0, float* dconv_hist, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* Training pair (saved intermediates).  prism_forward_train computes what
 * prism_forward computes and also keeps, in the caller-owned `saved` buffer,
 * the intermediates the backward needs: the refinement pairs (k^(l), w^(l))
 * of every token, and per chunk the affine map M^T, the decay sum g_C, the
 * chunk-entry state S_c, the readout operand Qt and the solve results U^T,
 * W_k^T (summary §2.1-2.2 as rewritten per chunk).  prism_backward_train then
 * returns the same gradients as prism_backward with the same inputs, starting
 * from those intermediates instead of recomputing the forward.
 *   saved:     device buffer of prism_saved_bytes() bytes, 256-byte aligned,
 *              written by prism_forward_train, read by prism_backward_train;
 *              the caller keeps it unchanged in between (same desc, same
 *              inputs, the same conv_hist contents, so not one that
 *              conv_hist_out overwrote; the backward does not check this).
 *   workspace: 256-byte aligned, prism_forward_train_workspace() /
 *              prism_backward_train_workspace() bytes.
 * Errors: as for the plain entry points; a NULL, misaligned or too small
 * `saved` buffer gives PRISM_ERR_WORKSPACE / PRISM_ERR_ALIGN before any HIP
 * call. */
prism_status prism_saved_bytes(const prism_desc* desc, size_t* bytes);
prism_status prism_forward_train(const prism_desc* desc, const void* q, const void* k,
                                 const void* v, const float* alpha, const float* beta,
                                 const void* Wk, const void* Wp, const void* wbeta,
                                 const void* conv, const float* S0, const void* conv_hist,
                                 const int* cu_seqlens, void* o, float* ST, void* conv_hist_out,
                                 void* saved, size_t saved_bytes, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);
prism_status prism_backward_train(const prism_desc* desc, const void* q, const void* k,
                                  const void* v, const float* alpha, const float* beta,
                                  const void* Wk, const void* Wp, const void* wbeta,
                                  const void* conv, const float* S0, const void* conv_hist,
                                  const int* cu_seqlens, const void* saved, size_t saved_bytes,
                                  const void* dO, const float* dST, void* dq, void* dk, void* dv,
                                  float* dalpha, float* dbeta, float* dWk, float* dWp,
                                  float* dwbeta, float* dconv, float* dS0, float* dconv_hist,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Recurrent form: the layer token by token (summary §2.1 S_t = S_{t-1} A_t
 * + B_t with §2.2's B_t, then o_t = S_t q_t), for the desc->T tokens of each
 * sequence in order.  With T = 1 this is the decode step of serving.
 *   S:          [B, H, dv, dk] f32, required, read as S_0 and overwritten
 *               with S_T (in place).
 *   conv_state: [B, 4, H, dv] dt, read as the ShortConv history before the
 *               tokens and overwritten with the history after them (in
 *               place); NULL means zeros, and nothing is written.
 *   o:          [B, T, H, dv] dt.
 *   workspace:  prism_step_workspace() bytes, 256-byte aligned (the
 *               refinement pairs of the tokens; 0 bytes and NULL allowed
 *               when L = 0).
 * The other inputs and desc fields are those of prism_forward; desc->chunk
 * must be valid but is not used.  A prism_forward over the first tokens
 * with ST and conv_hist_out, then prism_step over the rest, equals one
 * prism_forward over all of them up to rounding.  The state stays in
 * registers between tokens (one workgroup per sequence and head), so S
 * crosses HBM once per call.  Errors: as prism_forward. */
prism_status prism_step_workspace(const prism_desc* desc, size_t* bytes);
prism_status prism_step(const prism_desc* desc, const void* q, const void* k, const void* v,
                        const float* alpha, const float* beta, const void* Wk, const void* Wp,
                        const void* wbeta, const void* conv, float* S, void* conv_state, void* o,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* prism_step without a workspace, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, results and errors as prism_step,
 * except that the refinement pairs of the tokens go to a fixed device array
 * inside the library instead of a caller workspace:
 *   - the array holds 16 MiB per GPU (2 * B * H * L * T * dv elements of dt,
 *     each half rounded up to 256 bytes, must fit; e.g. B = 512, H = 16,
 *     L = 3, T = 1, dv = 128 in bf16); a larger call returns
 *     PRISM_ERR_WORKSPACE before any HIP call;
 *   - each GPU the library runs on keeps its own copy until the process
 *     ends; the call uses the copy of the device `stream` belongs to;
 *   - nothing is allocated or freed (no hipMalloc, hipFree or allocating
 *     library call): every pair the state kernel reads is written first by
 *     the same call, so the array needs no clearing between calls;
 *   - calls that overlap in time on one GPU (different streams, or several
 *     threads) share the array and race: serialise them. */
prism_status prism_step_noalloc(const prism_desc* desc, const void* q, const void* k,
                                const void* v, const float* alpha, const float* beta,
                                const void* Wk, const void* Wp, const void* wbeta,
                                const void* conv, float* S, void* conv_state, void* o,
                                hipStream_t stream);

/* Human-readable name of a status code (static string). */
const char* prism_status_string(prism_status status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* prism_last_error(void);

/* Kernel timing.  Between prism_timing_begin() and prism_timing_end(), every
 * kernel the library enqueues is bracketed by two HIP events recorded on the
 * stream it runs on.  prism_timing_end() waits for those events and fills up
 * to `capacity` entries: names[i] (static strings), total_ms[i] (sum of the
 * event-measured durations) and launches[i]; it returns the number of
 * distinct kernels.  Not thread-safe; meant for benchmarks. */
void prism_timing_begin(void);
int prism_timing_end(const char** names, double* total_ms, int* launches, int capacity);

#ifdef __cplusplus
}
#endif

#endif /* PRISM_H_ */

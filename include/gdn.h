/*
 * gdn.h -- C ABI of libgdn, the MI355X (gfx950) gated delta-rule library.
 *
 * The method: per head, a d_k x d_v associative state S is carried over the
 * sequence and updated by a gated delta rule,
 *
 *     S_t = alpha_t (I - beta_t k_t kread_t^T) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = S_t^T qread_t,
 *
 * where kread = k, qread = q for real data and kread = conj(k), qread = conj(q)
 * for complex data.  References for each piece:
 *   - rank-one delta write with a keyed readout and residual error:
 *     DeltaPhase README, section 2 "Complex Phase Matrix Delta Memory";
 *   - the data-dependent forget gate alpha_t: Sykra 0.3.3 README,
 *     "Architectural Highlights" (data-dependent forget gating); the gate
 *     scales the whole updated state (Gated DeltaNet ordering, named in the
 *     DeltaPhase lineage list);
 *   - beta in (0, 2) as the extended Householder range: DeltaPhase README,
 *     section 1 "Extended Householder Beta Range";
 *   - the chunkwise-parallel evaluation (WY / unit triangular transform) that
 *     gdn_chunk_fwd implements: Sykra README, "Architectural Highlights"
 *     (chunkwise parallel training), DeltaPhase README, section 1 "Fast
 *     Triangular Solve", and section 5 (log-space factorisation of the decay);
 *   - the O(d^2) single-token step of gdn_recurrent_step: Sykra README,
 *     "Computational Complexity" table (inference step time O(d^2), fixed state).
 * Around that forward: gdn_chunk_fwd_prologue folds the layer's input
 * transforms (L2 norms, gate logits) into it; gdn_chunk_bwd returns its
 * gradients; gdn_fwd_channel_decay replaces the scalar gate with a decay per
 * value channel (DeltaPhase README, section 5).
 *
 * Conventions shared by every entry point
 *   - All pointers are DEVICE pointers (memory the caller allocated on the
 *     current HIP device), except where stated.  The library allocates
 *     nothing and keeps no state besides a cached device-property query.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL means the null
 *     stream) and the call returns without synchronising.
 *   - Argument errors are reported synchronously, before anything is
 *     launched, and no output is touched.  A launch failure returns
 *     GDN_ERR_HIP.  Faults during execution surface at the caller's next
 *     synchronisation of the stream.  No C++ exception crosses this ABI.
 *   - Calls are thread-safe.  Two calls that write the same buffers must be
 *     ordered by the caller.
 *   - Element types: `dtype` selects the storage of q, k, v and out:
 *       GDN_F32  float32, GDN_BF16 bfloat16, GDN_C64 complex64 (interleaved
 *       re, im float32).  alpha and beta are always float32.  States (S0,
 *       S_final, S) are float32, or complex64 when dtype == GDN_C64.
 *       Gradients from gdn_chunk_bwd are float32.
 *   - Every pointer must be 16-byte aligned.
 *   - Size limits (GDN_ERR_SHAPE otherwise): no tensor above 2^40 elements;
 *     B * H below 2^20 for the chunk forwards, below 2^23 for the backward,
 *     below 2^22 for the channel-decay forward; N below 2^24 for the decode
 *     step.  These keep every launch under 2^32 work-items.
 *   - Preconditions not checked on the device (violations give undefined,
 *     typically non-finite, results): 0 < alpha <= 1, 0 <= beta <= 2, finite
 *     inputs.  Inputs and outputs must not overlap, except that S_final may
 *     equal S0.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum {
  GDN_OK = 0,
  GDN_ERR_NULL = 1,        /* a required pointer is NULL                     */
  GDN_ERR_SHAPE = 2,       /* a size is negative or the total is too large   */
  GDN_ERR_DTYPE = 3,       /* dtype is not one of GDN_F32, GDN_BF16, GDN_C64 */
  GDN_ERR_UNSUPPORTED = 4, /* valid but not supported (chunk, head dims)     */
  GDN_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned              */
  GDN_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required     */
  GDN_ERR_HIP = 7          /* the HIP runtime reported an error on launch    */
};

/* Element types (the `dtype` argument). */
enum { GDN_F32 = 0, GDN_BF16 = 1, GDN_C64 = 2 };

/*
 * Bytes of device workspace gdn_chunk_fwd needs for these sizes; 0 means the
 * call may pass workspace = NULL.  Returns 0 also for unsupported arguments
 * (gdn_chunk_fwd then reports the error).
 *
 * GDN_BF16 and GDN_F32 need none.  GDN_C64 needs B * H * ceil(T / 64) * 57600
 * bytes: per chunk the factors -W and U, (diag(lambda) K)^T, the decay
 * prefix and the chunk-start state, handed between its three launches.  The
 * caller owns the workspace; its contents are scratch on entry and exit.  Two
 * calls may share one workspace only if they are ordered (same stream).
 */
size_t gdn_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, int dtype);

/*
 * Chunkwise-parallel forward of the gated delta rule over whole sequences.
 *
 *   q, k      [B, T, H, dk]  dtype          queries and keys (row-major, d fastest)
 *   v         [B, T, H, dv]  dtype          values
 *   alpha     [B, T, H]      float32        forget gate, 0 < alpha <= 1
 *   beta      [B, T, H]      float32        write strength, 0 <= beta <= 2
 *   S0        [B, H, dk, dv] state type     initial state (row = key dim); NULL -> zeros
 *   chunk                                    chunk length C; 64 is supported
 *   out       [B, T, H, dv]  dtype          o_t for every token
 *   S_final   [B, H, dk, dv] state type     state after token T-1; NULL -> not written;
 *                                            may be the same buffer as S0
 *   workspace, workspace_bytes               device scratch, at least
 *                                            gdn_chunk_fwd_workspace_bytes(...) bytes
 *   stream                                   hipStream_t to enqueue on
 *
 * Supported: chunk == 64; dk == dv in {64, 128} for GDN_BF16; dk == dv == 64
 * for GDN_F32; dk == dv == 32 for GDN_C64.  Any T >= 0 (T % 64 != 0 is handled exactly:
 * the tail chunk is shorter).  B == 0, H == 0 or T == 0 with S_final given
 * copies S0 (or zeros) into S_final.
 *
 * Arithmetic: bf16 inputs are multiplied on bf16 matrix cores with fp32
 * accumulation; the state is carried in fp32.  fp32 and complex64 inputs use
 * fp32 matrix cores throughout.
 */
int gdn_chunk_fwd(const void *q, const void *k, const void *v, const float *alpha, const float *beta,
                  const void *S0, int chunk, void *out, void *S_final, int B, int T, int H, int dk,
                  int dv, int dtype, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace gdn_chunk_fwd_prologue needs for these sizes (0:
 * workspace may be NULL; 0 also for unsupported arguments).  bf16: 0 where
 * gdn_chunk_fwd needs no workspace; otherwise (the two-launch path) what
 * gdn_chunk_fwd needs plus B * H * ceil(T / 64) * 256 bytes, the inverse key
 * norms handed from the first launch to the second.  GDN_F32 and GDN_C64: the
 * transformed q and k (B * T * H rows of 256 bytes each) and the two gates
 * (B * T * H floats each), each rounded up to 256 bytes, plus, for GDN_C64,
 * what gdn_chunk_fwd needs.  Ownership and sharing as for gdn_chunk_fwd.
 */
size_t gdn_chunk_fwd_prologue_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, int dtype);

/*
 * gdn_chunk_fwd for a layer's raw projections, with its input transforms
 * applied on the device:
 *
 *   q_t <- q_t / max(|q_t|, 1e-12),  k_t <- k_t / max(|k_t|, 1e-12)
 *          (L2 over the key dimension, per token and head; the unit-norm keys
 *          and queries the chunkwise form is usually run on; for complex
 *          rows the Hermitian norm, sum over i of |q_i|^2)
 *   beta_t  = beta_scale * sigmoid(b_t)
 *          (DeltaPhase README, section 1 "Extended Householder Beta Range":
 *          beta_scale = 2 gives beta in (0, 2); 1 gives (0, 1))
 *   alpha_t = exp(-softplus(a_t)) = 1 / (1 + e^{a_t})
 *          (the data-dependent forget gate of the Sykra README, "Architectural
 *          Highlights", as a logistic map of a logit into (0, 1))
 *
 *   q, k      [B, T, H, dk]  dtype      raw queries and keys
 *   v         [B, T, H, dv]  dtype      values
 *   a_logit   [B, T, H]      float32    forget-gate logits
 *   b_logit   [B, T, H]      float32    write-strength logits
 *   beta_scale                          finite, 0 <= beta_scale <= 2
 *   workspace  device memory of at least
 *              gdn_chunk_fwd_prologue_workspace_bytes(...) bytes, or NULL when
 *              that is 0
 *   S0, chunk, out, S_final, B, T, H, dk, dv, dtype, stream: as for
 *   gdn_chunk_fwd.
 *
 * Supported: the shapes gdn_chunk_fwd supports (bf16 d = 64 or 128, fp32
 * d = 64, complex64 d = 32; dk == dv; chunk == 64), except bf16 shapes with a
 * batch row of q, k, v or out of 2^31 bytes or more, and bf16 d = 128 grids of
 * 2^26 chunks (B * H * ceil(T / 64)) or more (GDN_ERR_UNSUPPORTED).
 *
 * bf16 fuses the transforms into the forward's kernels, so q, k and the
 * logits are read once, as stored, and the rows are never rewritten: 1/|k|
 * and 1/|q| scale the Gram tiles, the decay factors and the per-token gates
 * (on the two-launch path, d = 128 and long d = 64 sequences, the first
 * launch forms both and the second reads them).  fp32 and complex64
 * run one extra pass over the rows that writes the transformed q, k and gates
 * to the workspace; there alpha is kept at or above 2^-126 (a logit above 87
 * already gives a gate that wipes the state).
 */
int gdn_chunk_fwd_prologue(const void *q, const void *k, const void *v, const float *a_logit,
                           const float *b_logit, float beta_scale, const void *S0, int chunk, void *out,
                           void *S_final, int B, int T, int H, int dk, int dv, int dtype, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * Bytes of workspace gdn_chunk_bwd needs.  bf16 (the chunk form): per
 * (chain, 64-token chunk) two 6400-byte factor records, a bf16 start state and
 * a bf16 end gradient (2 * 6400 + 2 * 64 * 64 * 2 bytes), plus the forward's
 * segment maps when it splits long sequences (as gdn_chunk_fwd_workspace_bytes
 * reports them).  fp32 (d = 64) and complex64 (d = 32): the forward state
 * every 8 tokens, B * H * ceil(T / 8) * d * d * e bytes (e = 4 or 8), plus the
 * shares of dq, dk, dalpha and dbeta from each of the n column groups (n = 8:
 * d / 8 for fp32, d / 4 for complex64), n * B * T * H * (2 * d * e + 8) bytes.
 * 0 for an unsupported combination.
 */
size_t gdn_chunk_bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int dtype);

/*
 * Reverse-mode gradients of gdn_chunk_fwd: given the gradients grad_out of
 * out and grad_S_final of S_final, the gradients of the real loss
 * sum(out * grad_out) + sum(S_final * grad_S_final) with respect to q, k, v,
 * alpha, beta and S0.  For complex data the loss is
 * Re sum(conj(grad_out) out) + Re sum(conj(grad_S_final) S_final), and the
 * gradient of a complex value z is dL/dRe(z) + i dL/dIm(z) (the upstream
 * gradients are given the same way); alpha and beta stay real.  The forward is the recurrence of DeltaPhase README
 * section 2 with the data-dependent forget gate of the Sykra README
 * ("Architectural Highlights"), applied to the whole Householder-updated
 * state, as for gdn_chunk_fwd; the gradients follow it token by token in
 * reverse.  The pages train through this layer; they print no gradient
 * formula.
 *
 *   q, k, v, alpha, beta, S0   the forward's inputs, as for gdn_chunk_fwd
 *                              (S0 may be NULL: zero)
 *   grad_out      [B, T, H, dv]  dtype     gradient of out
 *   grad_S_final  [B, H, dk, dv] float32 (complex64 for GDN_C64)   gradient
 *                 of S_final (NULL: zero)
 *   grad_q, grad_k [B, T, H, dk], grad_v [B, T, H, dv]   float32 (complex64
 *                 for GDN_C64), written
 *   grad_alpha, grad_beta [B, T, H]                      float32, written
 *   grad_S0       [B, H, dk, dv] float32 (complex64 for GDN_C64), written
 *                 (NULL: not computed)
 *   (for GDN_C64 the float pointers hold complex64 as interleaved re, im)
 *   workspace     device memory of at least gdn_chunk_bwd_workspace_bytes(...)
 *                 bytes, owned by the caller, overwritten (may be NULL when
 *                 that is 0)
 *
 * Supported: GDN_F32 with dk == dv == 64, GDN_BF16 with dk == dv == 64 or
 * 128, GDN_C64 with dk == dv == 32, any T >= 0 with T * H * 4 < 2^31;
 * otherwise GDN_ERR_UNSUPPORTED.
 * bf16 inputs take the chunk form on the matrix cores (the same chunking as
 * gdn_chunk_fwd, run in reverse: the forward's chunk start states, then the
 * gradient carried from the last chunk to the first, then every chunk's
 * gradients at once), with bf16 operands and fp32 accumulation, like the
 * forward.  fp32 and complex64 inputs take a token-by-token reverse pass in
 * fp32 throughout (checkpoints every 8 tokens), split by groups of state
 * columns, 8 for fp32 and 4 for complex64 (the columns evolve independently;
 * a second launch adds the groups' shares of dq, dk, dalpha and dbeta).  The forward is recomputed inside the call, so
 * nothing from a forward call is needed.  Gradient outputs must not alias any
 * input.  alpha must be positive (the chunk form works with log alpha).
 * B * H == 0 is a no-op; T == 0 copies grad_S_final (or zeros) to grad_S0.
 * Errors as for gdn_chunk_fwd.
 */
int gdn_chunk_bwd(const void *q, const void *k, const void *v, const float *alpha, const float *beta,
                  const float *S0, const void *grad_out, const float *grad_S_final, float *grad_q,
                  float *grad_k, float *grad_v, float *grad_alpha, float *grad_beta, float *grad_S0,
                  int B, int T, int H, int dk, int dv, int dtype, void *workspace,
                  size_t workspace_bytes, void *stream);

/*
 * The forward with a per-output-channel decay in place of the scalar gate,
 * LaplacePhaseCore's gated-decay rule (DeltaPhase README, section 2: the
 * memory is read through the key BEFORE it decays, and the error is written
 * along the key; section 5: the decay diag(r_t) sits on the memory's output
 * rows, one factor per value channel).  With S [dk, dv] (row = key dim),
 * for every value channel j:
 *
 *   e_t[j] = v_t[j] - kr_t^T s_j,   s_j <- r_t[j] s_j + beta_t k_t e_t[j],
 *   o_t[j] = qr_t^T s_j            (the updated state)
 *
 * with kr = k, qr = q for real data and kr = conj(k), qr = conj(q) for
 * complex data (LaplacePhaseCore's keys are complex, e^{s dt}), i.e.
 * S_t = S_{t-1} diag(r_t) + beta_t k_t (v_t - S_{t-1}^T kr_t)^T.  With every
 * r_t[j] = 1 it is gdn_chunk_fwd at alpha = 1.  (With r < 1 it differs from
 * gdn_chunk_fwd's ordering, where the gate also scales the erased part.)
 *
 *   q, k     [B, T, H, dk]  dtype    keys of norm <= 1 for a stable update
 *   v        [B, T, H, dv]  dtype
 *   r        [B, T, H, dv]  float32  decay per token and value channel, in (0, 1]
 *   beta     [B, T, H]      float32
 *   S0       [B, H, dk, dv] state    may be NULL (zero)
 *   out      [B, T, H, dv]  dtype, written
 *   S_final  [B, H, dk, dv] state, written; may be NULL, may equal S0
 *
 * The state is float32 for real data and complex64 (interleaved re, im) for
 * GDN_C64.  Supported: dtype GDN_F32 or GDN_BF16 with dk == dv == 64, or
 * GDN_C64 with dk == dv == 32, any T >= 0; otherwise GDN_ERR_UNSUPPORTED.
 * fp32 arithmetic.  No workspace.  B * H == 0
 * is a no-op; T == 0 copies S0 (or zeros) to S_final.  Errors as for
 * gdn_chunk_fwd.
 */
int gdn_fwd_channel_decay(const void *q, const void *k, const void *v, const float *r, const float *beta,
                          const float *S0, void *out, float *S_final, int B, int T, int H, int dk, int dv,
                          int dtype, void *stream);

/*
 * gdn_chunk_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and results as gdn_chunk_fwd, without the workspace: the
 * call takes it from a fixed device array that the library keeps per device,
 * from the first call on that device until the process ends.  The call
 * itself allocates nothing (no hipMalloc, hipFree or allocating library
 * routine).
 *
 * Limit: GDN_NOALLOC_MAX_WORKSPACE bytes (128 MiB), compared with
 * gdn_chunk_fwd_workspace_bytes(...) for the same sizes; a call that needs
 * more returns GDN_ERR_WORKSPACE before anything is launched.  Calls that need
 * no workspace (fp32, and bf16 d = 64 with enough chains) use none.
 *
 * All calls on one device share the array: calls that may overlap on one
 * device (different streams, unordered host threads) race and give wrong
 * results.  Order them (one stream) or use gdn_chunk_fwd with a workspace of
 * your own.  Other errors as for gdn_chunk_fwd; GDN_ERR_HIP if the array's
 * device address cannot be found.
 */
int gdn_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const float *alpha,
                          const float *beta, const void *S0, int chunk, void *out, void *S_final,
                          int B, int T, int H, int dk, int dv, int dtype, void *stream);
#define GDN_NOALLOC_MAX_WORKSPACE ((size_t)128 << 20)

/*
 * One single-token decode step on N independent states, in place.
 *
 *   q, k   [N, dk] dtype;  v [N, dv] dtype;  alpha, beta [N] float32
 *   S      [N, dk, dv] state type, read and overwritten with the new state
 *   out    [N, dv] dtype, o = S_new^T qread
 *
 * Supported: dk == dv == 64 or 128 for GDN_F32 / GDN_BF16; 32 for GDN_C64.
 * N == 0 is a no-op.  The state is read once and written once.
 */
int gdn_recurrent_step(const void *q, const void *k, const void *v, const float *alpha,
                       const float *beta, void *S, void *out, int N, int dk, int dv, int dtype,
                       void *stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *gdn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */

/*
 * kla.h -- C ABI of libkla: the Kalman Linear Attention (KLA) scan on AMD
 * Instinct MI355X (gfx950) -- forward pass, its backward pass, the fused
 * mixer (forward and backward), the time-invariant-gate form and the
 * one-token decode steps of the scan and of the mixer.
 *
 * The operation (Pith review of arXiv 2602.10743, "What carries the
 * argument" and "Circularity check"; "KLA Part 1" primer, sections 2 and
 * 5.1).  Every channel (b, h, d) of a [B, H, T, D] tensor runs its own scalar
 * Kalman filter in information form.  With the posterior precision lam and
 * information mean eta before the first token given by lam0, eta0, each token
 * t = 1..T applies
 *
 *     predict:  lam_prior = lam_{t-1} / (a_t^2 + p_t lam_{t-1})
 *     update:   lam_t     = lam_prior + phi_t
 *     mean:     eta_t     = f_t eta_{t-1} + b_t,
 *               f_t       = a_t / (a_t^2 + p_t lam_{t-1})
 *
 * i.e. lam_t = M_t(lam_{t-1}) is the Moebius map of the 2x2 matrix
 * M_t = [[1 + p_t phi_t, a_t^2 phi_t], [p_t, a_t^2]] and eta follows an
 * affine recursion whose forget gate is the precision ratio.  a_t is the
 * state decay, p_t the process-noise variance, phi_t the precision of the
 * token's evidence and b_t its information (phi_t times the observed value).
 * Both recursions are associative, so the library evaluates them as a
 * chunked parallel scan; the result equals the sequential filter up to
 * rounding.
 *
 * Outputs: lam[..., t-1, :] and eta[..., t-1, :] hold lam_t and eta_t, the
 * posterior after token t.  The last time row is the final state: passing it
 * as lam0/eta0 of a following call continues the same sequence.
 */
#ifndef KLA_H
#define KLA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#if defined(__GNUC__) || defined(__clang__)
#define KLA_API __attribute__((visibility("default")))
#else
#define KLA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KLA_OK = 0,
    KLA_ERR_INVALID_ARG = 1,  /* null pointer, negative size, overflow, aliasing */
    KLA_ERR_UNSUPPORTED = 2,  /* dtype or alignment the library does not handle */
    KLA_ERR_WORKSPACE = 3,    /* workspace missing, too small or misaligned */
    KLA_ERR_HIP = 4           /* the HIP runtime reported an error */
} kla_status;

typedef enum {
    KLA_DTYPE_F32 = 0,  /* IEEE binary32 */
    KLA_DTYPE_BF16 = 1  /* bfloat16 (upper half of a binary32) */
} kla_dtype;

/*
 * Bytes of device workspace kla_scan_fwd needs for this problem.  Returns 0
 * when the sizes are invalid (negative or overflowing) or when the problem is
 * empty (some size is 0, so there is nothing to do).
 */
KLA_API size_t kla_scan_fwd_workspace_size(int64_t B, int64_t H, int64_t T, int64_t D,
                                   kla_dtype in_dtype);

/*
 * Forward KLA scan.
 *
 *   a, p, phi, b  device pointers, [B, H, T, D] row-major (D fastest), all of
 *                 dtype in_dtype; naturally aligned (4 B for f32, 2 B for bf16).
 *                 Domain: a > 0, p >= 0, phi >= 0, all finite, and every
 *                 per-token factor (1 + p phi, a^2 phi, |b| p, |b| a^2) below
 *                 2^120.  Outside it the results are unspecified; NaN inputs
 *                 propagate.
 *   lam0, eta0    device pointers, [B, H, D] float32: the posterior precision
 *                 (> 0) and information mean before the first token.  Either
 *                 may be NULL, meaning lam0 = 1 and eta0 = 0 for every channel.
 *   lam, eta      device pointers, [B, H, T, D] float32 outputs, 4-B aligned.
 *                 They must not overlap each other, an input or the workspace.
 *                 Values whose float32 rounding overflows are written as
 *                 +-infinity.
 *   B, H, T, D    sizes.  If any is 0 the call does nothing and returns KLA_OK.
 *   workspace     device memory of at least kla_scan_fwd_workspace_size(...)
 *                 bytes, 256-B aligned, owned by the caller.  It must be
 *                 zero-filled before its first use; every call leaves it ready
 *                 for the next one, so it is zeroed once, not per call.  Calls
 *                 that run at the same time must use different workspaces.
 *   stream        the HIP stream to enqueue on (NULL: the null stream).
 *
 * The call validates its arguments on the host and returns an error before
 * enqueueing anything (no partial writes).  On KLA_OK the work is enqueued
 * and runs asynchronously on `stream`; the caller keeps every buffer alive
 * until it completes.  The call allocates and frees nothing and uses no
 * library-held state; it is re-entrant and thread-safe.
 */
KLA_API kla_status kla_scan_fwd(const void *a, const void *p, const void *phi,
                        const void *b, kla_dtype in_dtype,
                        const float *lam0, const float *eta0,
                        float *lam, float *eta,
                        int64_t B, int64_t H, int64_t T, int64_t D,
                        void *workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * kla_scan_fwd without a caller-owned workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, results, errors and
 * stream semantics as kla_scan_fwd, with the same kernels; the workspace is a
 * device array inside the library, kla_scan_fwd_noalloc_max_workspace()
 * bytes (32 MiB) per GPU, which each GPU holds from its first call until the
 * process ends (its address is resolved once per device on that device's
 * first call, with that device current).  The call itself allocates and
 * frees nothing and clears nothing: the array starts zero-filled and every
 * call leaves it ready for the next one.
 *
 * Limit: a problem whose kla_scan_fwd_workspace_size exceeds the array is
 * rejected with KLA_ERR_WORKSPACE before anything is enqueued (about 7,000
 * tiles of 64 channels by 112 float32 rows, e.g. 52M float32 elements at
 * D = 64).  All calls on one GPU share its array: calls that may overlap in
 * time on one GPU (different streams or threads) race and must be serialised
 * by the caller.
 */
KLA_API size_t kla_scan_fwd_noalloc_max_workspace(void);
KLA_API kla_status kla_scan_fwd_noalloc(const void *a, const void *p, const void *phi,
                                        const void *b, kla_dtype in_dtype,
                                        const float *lam0, const float *eta0,
                                        float *lam, float *eta,
                                        int64_t B, int64_t H, int64_t T, int64_t D,
                                        hipStream_t stream);

/*
 * Bytes of device workspace kla_scan_bwd needs (0 for invalid sizes or an
 * empty problem).  A workspace large enough for both directions may serve
 * forward and backward calls alternately.
 */
KLA_API size_t kla_scan_bwd_workspace_size(int64_t B, int64_t H, int64_t T, int64_t D,
                                           kla_dtype in_dtype);

/*
 * Backward KLA scan: the vector-Jacobian product of kla_scan_fwd.
 *
 * Reverse-mode differentiation of the forward step (Pith review of arXiv
 * 2602.10743, "Circularity check", Theorems 1 and 2).  With
 * d_t = a_t^2 + p_t lam_{t-1} and upstream gradients g_lam, g_eta of a scalar
 * loss with respect to the outputs lam, eta, it returns the loss gradients
 * with respect to every input:
 *     g_phi[t] = Lam_t,  g_b[t] = Eta_t   (total adjoints of lam_t, eta_t)
 *     g_a[t] = Lam_t (-2 a lam_{t-1}) / d^2 + Eta_t eta_{t-1} (p lam_{t-1} - a^2) / d^2
 *     g_p[t] = -lam_{t-1} (Lam_t lam_{t-1} + Eta_t a eta_{t-1}) / d^2
 *     Lam_{t-1} = g_lam[t-1] + (a/d)^2 Lam_t - p (a/d) eta_{t-1} / d Eta_t,
 *     Eta_{t-1} = g_eta[t-1] + (a/d) Eta_t,
 * and g_lam0, g_eta0 are the adjoints carried past the first token.  It runs
 * as the same single-pass scan as the forward call, from the end of the
 * sequence.
 *
 *   a, p          the forward call's gates, [B,H,T,D] of in_dtype (phi and b
 *                 are not needed).
 *   lam0, eta0    the forward call's initial state ([B,H,D] float32 or NULL).
 *   lam, eta      the forward call's outputs, [B,H,T,D] float32: they are the
 *                 states lam_{t-1}, eta_{t-1} of the derivatives, so they must
 *                 be finite (where the forward outputs overflowed float32 the
 *                 gradients are unspecified; kla_scan_bwd_states below has
 *                 no such limit).
 *   g_lam, g_eta  upstream gradients, [B,H,T,D] float32; NULL means zero.
 *   g_a, g_p, g_phi, g_b   outputs, [B,H,T,D] float32 (also for bf16 gates).
 *   g_lam0, g_eta0         outputs, [B,H,D] float32; either may be NULL.
 *   workspace, stream      as for kla_scan_fwd (same zero-once contract).
 * Outputs must not overlap any other argument.  Errors as for kla_scan_fwd.
 */
KLA_API kla_status kla_scan_bwd(const void *a, const void *p, kla_dtype in_dtype,
                                const float *lam0, const float *eta0,
                                const float *lam, const float *eta,
                                const float *g_lam, const float *g_eta,
                                float *g_a, float *g_p, float *g_phi, float *g_b,
                                float *g_lam0, float *g_eta0,
                                int64_t B, int64_t H, int64_t T, int64_t D,
                                void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The backward pass from float64 states: the vector-Jacobian product of
 * kla_scan_fwd (the same gradients as kla_scan_bwd), defined wherever the
 * forward recursion is, also where lam or eta leave float32's range.
 *
 * kla_scan_bwd takes its states lam_{t-1}, eta_{t-1} from the forward
 * outputs, which are float32: where those overflow (lam reaches 1e88 on
 * hard gates) its gradients are unspecified.  These entry points keep the
 * states in float64 instead: the forward call writes the state (lam, eta)
 * of every channel after every 8th token, and the backward kernel replays
 * each 8-token block from the state before it in float64.
 *
 * kla_scan_states_size: bytes of the `states` buffer, 16 per channel per 8
 * tokens ([ceil(T / 8)][B * H * D][2] float64), about 2 bytes per element;
 * 0 for an empty or overflowing problem.
 *
 * kla_scan_fwd_states: kla_scan_fwd (same arguments, outputs, workspace
 * and errors) that also writes `states` (device pointer, 16-byte aligned,
 * kla_scan_states_size bytes, not overlapping any other argument).
 *
 * kla_scan_bwd_states: the gradients of a scalar loss with respect to a, p,
 * phi, b (per token) and lam0, eta0, given the upstream gradients g_lam,
 * g_eta of the forward outputs (formulas as for kla_scan_bwd).
 *   a, p, phi, b, lam0, eta0  the forward call's inputs.
 *   states         kla_scan_fwd_states' `states` for these inputs, or NULL:
 *                  the call then first recomputes them into the workspace
 *                  (one more pass over the gates).  Read only.
 *   g_lam, g_eta   [B, H, T, D] float32; NULL means zero.
 *   g_a, g_p, g_phi, g_b   [B, H, T, D] float32 outputs.
 *   g_lam0, g_eta0         [B, H, D] float32 outputs; either may be NULL.
 *   workspace      kla_scan_bwd_states_workspace_size bytes (it holds the
 *                  recomputed states), zero-filled once before first use as
 *                  for kla_scan_fwd; it may serve the other entry points in
 *                  turn.
 * Outputs must not overlap any other argument.  Errors, stream semantics and
 * the overflow rule as for kla_scan_fwd.
 */
KLA_API size_t kla_scan_states_size(int64_t B, int64_t H, int64_t T, int64_t D);
KLA_API kla_status kla_scan_fwd_states(const void *a, const void *p, const void *phi,
                                       const void *b, kla_dtype in_dtype,
                                       const float *lam0, const float *eta0,
                                       float *lam, float *eta, double *states,
                                       int64_t B, int64_t H, int64_t T, int64_t D,
                                       void *workspace, size_t workspace_bytes,
                                       hipStream_t stream);
KLA_API size_t kla_scan_bwd_states_workspace_size(int64_t B, int64_t H, int64_t T, int64_t D,
                                                  kla_dtype in_dtype);
KLA_API kla_status kla_scan_bwd_states(const void *a, const void *p, const void *phi,
                                       const void *b, kla_dtype in_dtype,
                                       const float *lam0, const float *eta0,
                                       const double *states,
                                       const float *g_lam, const float *g_eta,
                                       float *g_a, float *g_p, float *g_phi, float *g_b,
                                       float *g_lam0, float *g_eta0,
                                       int64_t B, int64_t H, int64_t T, int64_t D,
                                       void *workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/*
 * One decode step: advances a running filter state by one token, in place.
 *
 * For every channel i < n_channels (any layout; B*H*D channels of one token):
 *     d = a^2 + p lam,  lam <- lam / d + phi,  eta <- (a / d) eta + b,
 * the step of kla_scan_fwd (computed in float64, stored as float32), so that
 * repeated decode steps continue a sequence whose prefix went through
 * kla_scan_fwd (pass its last output row as the state).  This is the
 * linear-time inference of the "KLA Part 1" primer: constant work and memory
 * per token.
 *
 *   a, p, phi, b  device pointers, [n_channels] of in_dtype (same domain as
 *                 kla_scan_fwd).
 *   lam, eta      device pointers, [n_channels] float32, read and written.
 * No workspace; asynchronous on `stream`; errors as for kla_scan_fwd.
 */
KLA_API kla_status kla_decode_step(const void *a, const void *p, const void *phi,
                                   const void *b, kla_dtype in_dtype,
                                   float *lam, float *eta, int64_t n_channels, hipStream_t stream);

/*
 * One decode step of the fused mixer: the token step of kla_mixer_fwd for
 * every channel of one token, on a running state, in place.
 *
 * Channel i (i < n_channels = B*H*D, laid out as [B, H, D]) forms
 * phi = k^2 lam_v and b = k lam_v v from its token inputs, takes the gates
 * a, p of channel i % hd (hd = H*D), applies the step of kla_decode_step to
 * (lam, eta), and writes the readout out = q eta / lam and the variance
 * var = 1 / lam of the new state (computed in float64; the state is stored
 * back in float32).  Passing kla_mixer_fwd's lam_T, eta_T as the state
 * continues a sequence whose prefix went through kla_mixer_fwd.
 *
 *   k, v, lam_v, q  device pointers, [n_channels] of in_dtype.
 *   a, p            device pointers, [hd] float32.
 *   lam, eta        device pointers, [n_channels] float32, read and written.
 *   out             device pointer, [n_channels] float32, written.
 *   var             device pointer, [n_channels] float32, written; may be NULL.
 *   n_channels      a multiple of hd (0: no-op).
 * No workspace; asynchronous on `stream`; errors as for kla_scan_fwd.
 */
KLA_API kla_status kla_mixer_decode_step(const void *k, const void *v, const void *lam_v,
                                         const void *q, kla_dtype in_dtype,
                                         const float *a, const float *p,
                                         float *lam, float *eta, float *out, float *var,
                                         int64_t n_channels, int64_t hd, hipStream_t stream);

/*
 * Forward KLA scan for time-invariant gates (the linear time-invariant case
 * of the Pith review of arXiv 2602.10743, minor comment on Theorem 3, whose
 * convolutional form covers it).
 *
 * Same recursion and outputs as kla_scan_fwd, with a_t = a[h, d],
 * p_t = p[h, d], phi_t = phi[h, d] for every token: only the information b
 * is per token.  Then lam_t does not depend on the data, and from the
 * stationary precision lam* (the fixed point of the Moebius map) eta is the
 * causal convolution of b with the kernel f*^j, f* = a / (a^2 + p lam*).
 * For a scalar channel that geometric kernel is evaluated exactly by the
 * first-order recursion, so the library runs the scan with the gates read
 * once per channel: 12 bytes of HBM traffic per element (f32 b) instead of
 * 24.  Any initial state is allowed (the transient is exact too).
 *
 *   a, p, phi       device pointers, [H, D] float32 (a > 0, p >= 0, phi >= 0).
 *   b               device pointer, [B, H, T, D] of in_dtype.
 *   lam0, eta0, lam, eta, workspace, stream: as for kla_scan_fwd, with
 *   kla_scan_lti_fwd_workspace_size bytes of workspace.
 * Errors as for kla_scan_fwd.
 */
KLA_API size_t kla_scan_lti_fwd_workspace_size(int64_t B, int64_t H, int64_t T, int64_t D,
                                               kla_dtype in_dtype);
KLA_API kla_status kla_scan_lti_fwd(const float *a, const float *p, const float *phi,
                                    const void *b, kla_dtype in_dtype,
                                    const float *lam0, const float *eta0,
                                    float *lam, float *eta,
                                    int64_t B, int64_t H, int64_t T, int64_t D,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Fused KLA mixer forward: gate production, scan and readout in one pass.
 *
 * A KLA mixer channel observes its token value through an observation
 * operator k with a token-dependent value precision lam_v, under a state decay
 * a and process noise p that do not depend on the token (Pith review of arXiv
 * 2602.10743, "Circularity check": the update adds k^2 lam_v to the
 * precision; "Axiom & Free-Parameter Ledger": OU decay a learned and
 * time-invariant, process-noise scale p learned, value precision and the
 * observation/readout operators k, q produced from the input).  Per channel
 * (b, h, d) and token t:
 *
 *     phi_t = k_t^2 lam_v_t,   b_t = k_t lam_v_t v_t           (gates)
 *     (lam_t, eta_t) = the kla_scan_fwd step with a_t = a[h, d], p_t = p[h, d]
 *     out_t = q_t eta_t / lam_t   (readout of the posterior mean)
 *     var_t = 1 / lam_t           (posterior variance)
 *
 * i.e. the Kalman filter of x_t = a x_{t-1} + w_t (Var w_t = p),
 * v_t = k_t x_t + e_t (precision of e_t = lam_v_t), read out as q_t times the
 * posterior mean.  The gate tensors never exist in memory.  The discretised
 * OU decay (a = exp(-A delta)) is the caller's.
 *
 *   k, v, lam_v, q  device pointers, [B, H, T, D] of in_dtype; lam_v >= 0.
 *   a, p            device pointers, [H, D] float32; a > 0, p >= 0.
 *   lam0, eta0      as for kla_scan_fwd (NULL: 1 and 0).
 *   out             device pointer, [B, H, T, D] float32, written.
 *   var             device pointer, [B, H, T, D] float32, written; may be NULL.
 *   lam_T, eta_T    device pointers, [B, H, D] float32: the state after the
 *                   last token (pass it as lam0/eta0 of a following call);
 *                   both NULL or both given.
 *   states          device pointer, 16-byte aligned, kla_mixer_states_size
 *                   bytes, written; or NULL.  Receives the float64 pair
 *                   (lam, eta) of every channel after every 8th token
 *                   ([ceil(T / 8)][B * H * D][2]); a training caller keeps it
 *                   and hands it to kla_mixer_bwd, which then skips its
 *                   recompute of the forward states.
 *   workspace       kla_mixer_fwd_workspace_size bytes, same contract as for
 *                   kla_scan_fwd; one workspace large enough for each call
 *                   serves both entry points in turn.
 * Errors, stream semantics and the overflow rule as for kla_scan_fwd.
 */
KLA_API size_t kla_mixer_fwd_workspace_size(int64_t B, int64_t H, int64_t T, int64_t D,
                                            kla_dtype in_dtype);
KLA_API kla_status kla_mixer_fwd(const void *k, const void *v, const void *lam_v,
                                 const void *q, kla_dtype in_dtype,
                                 const float *a, const float *p,
                                 const float *lam0, const float *eta0,
                                 float *out, float *var, float *lam_T, float *eta_T,
                                 double *states,
                                 int64_t B, int64_t H, int64_t T, int64_t D,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream);
/* Bytes of kla_mixer_fwd's `states` output (0 for an empty or overflowing
 * problem): 16 bytes per channel per 8 tokens, about 2 bytes per element. */
KLA_API size_t kla_mixer_states_size(int64_t B, int64_t H, int64_t T, int64_t D);

/*
 * Fused KLA mixer backward: the vector-Jacobian product of kla_mixer_fwd.
 *
 * For a loss with upstream gradients g_out (of out) and g_var (of var),
 * returns the gradients of the token inputs, of the channel gates (summed
 * over the batch and the sequence) and of the initial state.  The readout
 * gives per token the adjoints d/dlam = -(g_out q eta + g_var) / lam^2 and
 * d/deta = g_out q / lam, which run through the reverse scan of
 * kla_scan_bwd (the review's Theorems 1 and 2 differentiated); the gate
 * adjoints reach k, v, lam_v through phi = k^2 lam_v and b = k lam_v v.
 * The backward kernel needs the float64 forward state after every 8th token
 * and replays the rows in between on chip.  Given `states` (kept by
 * kla_mixer_fwd on the same inputs) it uses them; with states NULL it first
 * recomputes them from the inputs into the workspace, so nothing needs
 * saving between the forward and backward calls.
 *
 *   k, v, lam_v, q, a, p, lam0, eta0   as passed to kla_mixer_fwd.
 *   states          device pointer, as written by kla_mixer_fwd for these
 *                   inputs, or NULL (recompute).  Read only.
 *   g_out           device pointer, [B, H, T, D] float32.
 *   g_var           device pointer, [B, H, T, D] float32, or NULL (zero).
 *   g_k, g_v, g_lam_v, g_q   device pointers, [B, H, T, D] float32, written.
 *   g_a, g_p        device pointers, [H, D] float32, written (sums over b, t
 *                   in a fixed order: deterministic).
 *   g_lam0, g_eta0  device pointers, [B, H, D] float32, written; may be NULL.
 *   workspace       kla_mixer_bwd_workspace_size bytes (it holds the
 *                   recomputed states: about 2 bytes per element), zero-filled
 *                   once before first use, as for kla_scan_fwd; it may also
 *                   serve the other entry points in turn.
 * A size-0 problem is a no-op.  Errors and stream semantics as for
 * kla_scan_fwd.
 */
KLA_API size_t kla_mixer_bwd_workspace_size(int64_t B, int64_t H, int64_t T, int64_t D,
                                            kla_dtype in_dtype);
KLA_API kla_status kla_mixer_bwd(const void *k, const void *v, const void *lam_v,
                                 const void *q, kla_dtype in_dtype,
                                 const float *a, const float *p,
                                 const float *lam0, const float *eta0,
                                 const double *states,
                                 const float *g_out, const float *g_var,
                                 float *g_k, float *g_v, float *g_lam_v, float *g_q,
                                 float *g_a, float *g_p, float *g_lam0, float *g_eta0,
                                 int64_t B, int64_t H, int64_t T, int64_t D,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Reads the workspace's health word after the calls that used it have
 * completed (it synchronizes `stream`).  *flags_out is 0 when every call so
 * far ran normally; bit 0 is set if a chunk gave up waiting for the carry of
 * its predecessor (the outputs of that call are then wrong).  Every wait is
 * bounded (about 2^20 polls), so a kernel always terminates; once one wait
 * of a call gives up, the other waits of the same call give up early, while
 * later calls wait normally.  The word is cleared by the read.  Returns
 * KLA_ERR_WORKSPACE for a NULL workspace.
 */
KLA_API kla_status kla_workspace_health(void *workspace, uint32_t *flags_out, hipStream_t stream);

/* Static text for a status code. */
KLA_API const char *kla_status_string(kla_status s);

/*
 * Thread-local text describing the last error the calling thread got from
 * this library (argument name, HIP error string), or "" if none.
 */
KLA_API const char *kla_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* KLA_H */

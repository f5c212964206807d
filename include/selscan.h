/*
 * libselscan -- the selective state-space scan (Mamba's selective SSM) on AMD
 * Instinct MI355X (gfx950).  Plain C ABI: device pointers, sizes, a HIP stream.
 *
 * The operation (all passages are on the reference pages):
 *
 *   Delta[b,l,d] = softplus(delta[b,l,d] + delta_bias[d])
 *       velog.io Mamba review, section 3.2 "Improving SSMs with Selection":
 *       the step is a projection plus a learned parameter passed through softplus,
 *       with shape (B, L, D); A has shape (D, N); B and C have shape (B, L, N).
 *   Abar = exp(Delta A),  Bbar = (Delta A)^-1 (exp(Delta A) - I) Delta B
 *       velog.io review, section "2 State Space Models", "Discretization"
 *       (zero-order hold; A is diagonal, so both are elementwise per (d, n):
 *       Bbar[b,l,d,n] = (exp(Delta A[d,n]) - 1) / A[d,n] * B[b,l,n], and
 *       Delta * B[b,l,n] in the limit A[d,n] = 0).
 *   h_l = Abar_l h_{l-1} + Bbar_l x_l,   y_l = C_l . h_l + D x_l,   y_l *= silu(z_l)
 *       velog.io review, "Discretization" item 3 (state and output equations);
 *       skip term and gate: gh.r-mj.com Mamba_Model_Report.md, sections 3
 *       (MambaBlock.forward: y * silu(z)) and 4.2 (y = y + D * x).
 *   Single-token recurrent step on a carried state [B, D, N]:
 *       Mamba_Model_Report.md, section 6 (ssm_step).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller, dense and
 *    row-major (last index fastest).  The library never frees or retains them.
 *  - Token tensors x, delta, z, y, and B, C use the element type `dtype`
 *    (SSCAN_F32 = float32, SSCAN_BF16 = bfloat16 stored as 16-bit words).
 *    A, D, delta_bias and every state tensor are float32.
 *  - Arithmetic is float32 in registers (state included); y is rounded to
 *    `dtype` with round-to-nearest-even.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null
 *    stream).  The library allocates no device memory and never synchronizes
 *    (sscan_fwd_noalloc's static scratch array comes with the loaded code object).
 *  - Errors: a nonzero sscan_status is returned and nothing is launched;
 *    sscan_last_error() gives a message (per calling thread).  Arguments are
 *    checked on the host before any launch.  Values are not checked: NaN and
 *    Inf propagate.  SSCAN_ERR_HIP reports a failed launch.
 *  - Outputs must not overlap inputs, except where stated (in-place state).
 *  - dstate (N) must be in [1, SSCAN_MAX_DSTATE]; seqlen at most SSCAN_MAX_SEQLEN.
 *  - `flags` selects variants of the method (SSCAN_FLAG_*); 0 is the method
 *    as defined above.
 */
#ifndef SELSCAN_H
#define SELSCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSCAN_VERSION 410
#define SSCAN_MAX_DSTATE 16
#define SSCAN_MAX_DCONV 4
/* Longest sequence sscan_fwd* and sscan_bwd* accept (2^30 steps): the kernels count
 * the steps of one sequence segment in 32-bit integers.  Longer ones are rejected
 * with SSCAN_ERR_INVALID_ARG. */
#define SSCAN_MAX_SEQLEN (1LL << 30)

/*
 * Bits of the `flags` argument.
 *
 * SSCAN_FLAG_EULER: discretize B with the first-order (Euler) rule
 *   Bbar = Delta * B   instead of the zero-order hold (Abar is exp(Delta A) either way).
 *   This is the rule the page-3 report's code uses (section 4.2,
 *   selective_scan / selective_scan_seq: deltaB = delta * B, BX = deltaB * x).
 * Unknown bits are rejected with SSCAN_ERR_UNSUPPORTED.
 */
#define SSCAN_FLAG_EULER 1u

/*
 * SSCAN_FLAG_STRUCTURED_A: the caller states that A is rank one, A[d, n] = c_d a_n --
 *   as the S4D-Real initialisation A = -(n + 1) of every channel (Mamba_Model_Report.md,
 *   section 3, MambaBlock: A = -exp(A_log) with A_log = log(1 .. N) for each channel).
 *   Then x B / A = (x / c_d)(B / a_n), and the forward stages x / c_d and B / a_n once
 *   per token instead of dividing per state.  A hint, never a change of the result:
 *   each channel tile checks the form exactly (c_d = A[d, 0], a_n = A[d0, n] / A[d0, 0]
 *   for the tile's first channel d0, and c_d a_n == A[d, n] with no rounding) and runs
 *   the plain form where it does not hold; results agree with the flag's absence to
 *   float32 rounding.  Used by sscan_fwd, sscan_fwd_segmented and sscan_fwd_noalloc with
 *   the zero-order hold when the launch takes the row layout (grids of at most one
 *   workgroup per compute unit); ignored otherwise and by the other entry points.
 */
#define SSCAN_FLAG_STRUCTURED_A 2u

typedef enum {
  SSCAN_OK = 0,
  SSCAN_ERR_INVALID_ARG = 1,  /* bad size, null required pointer, overlap, misalignment */
  SSCAN_ERR_UNSUPPORTED = 2,  /* dstate outside [1, SSCAN_MAX_DSTATE], unknown dtype   */
  SSCAN_ERR_HIP = 3           /* a HIP launch or runtime call failed                  */
} sscan_status;

typedef enum {
  SSCAN_F32 = 0,
  SSCAN_BF16 = 1
} sscan_dtype;

/* Library version (SSCAN_VERSION of the build). */
int sscan_version(void);

/* Message describing the last error returned to the calling thread ("" if none). */
const char* sscan_last_error(void);

/*
 * Workspace bytes that let sscan_fwd split long sequences into independently
 * scanned segments joined by a carry pass (a two-level scan over the sequence).
 * Returns 0 when the shape needs no split.  Pass at least this many bytes to
 * sscan_fwd to get the full split; fewer bytes give fewer segments (possibly
 * one), which is slower but equally correct.  The part of the workspace a call
 * uses must not overlap any tensor of that call (SSCAN_ERR_INVALID_ARG).
 */
size_t sscan_fwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                int dtype);

/*
 * Forward selective scan over whole sequences.
 *
 *   x, delta, z, y : [batch, seqlen, dim]     (dtype)
 *   A              : [dim, dstate]            (float32; real, normally negative)
 *   B, C           : [batch, seqlen, dstate]  (dtype)
 *   D, delta_bias  : [dim]                    (float32)
 *   initial_state  : [batch, dim, dstate]     (float32)
 *   last_state     : [batch, dim, dstate]     (float32) state after the last step
 *
 * Optional (NULL allowed): D (no skip term), z (no gate), delta_bias (zero),
 * initial_state (zero state), last_state (not written), workspace (no split).
 * last_state may be the same buffer as initial_state.
 * Result: y[b,l,d] as defined at the top of this header.  With seqlen == 0,
 * last_state receives the initial state (zeros when absent).
 * Alignment: dtype-size alignment for token tensors, 4 bytes for float32 ones.
 */
sscan_status sscan_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                       unsigned int flags, const void* x, const void* delta, const float* A, const void* B, const void* C,
                       const float* D, const void* z, const float* delta_bias,
                       const float* initial_state, void* y, float* last_state,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes that give sscan_fwd_segmented the split it asks for: num_segments
 * after the same clamping the call applies (to whole 16-step chunks of seqlen and at
 * least one segment).  num_segments == 0 gives sscan_fwd_workspace_size.  Returns 0
 * when that plan has one segment, or for a negative num_segments or an invalid shape.
 */
size_t sscan_fwd_segmented_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                          int dtype, int64_t num_segments);

/*
 * Same as sscan_fwd, with the number of sequence segments chosen by the caller
 * (num_segments >= 1; it is clamped to what the workspace and seqlen allow).
 * num_segments == 0 means "choose automatically" and equals sscan_fwd.
 * For tuning and testing the two-level split; results agree with sscan_fwd
 * up to float32 rounding.
 */
sscan_status sscan_fwd_segmented(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                                 unsigned int flags, const void* x, const void* delta, const float* A, const void* B,
                                 const void* C, const float* D, const void* z, const float* delta_bias,
                                 const float* initial_state, void* y, float* last_state,
                                 void* workspace, size_t workspace_bytes, int64_t num_segments,
                                 void* stream);

/*
 * sscan_fwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Arguments, results
 * and errors are those of sscan_fwd without the workspace; the two-level split's
 * scratch (carries, segment end states, step sums) lives instead in a static device
 * array of SSCAN_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs
 * on until the process ends.  The call allocates nothing (no hipMalloc, no
 * allocating library routine).  It chooses the same split as sscan_fwd with a
 * workspace of sscan_fwd_workspace_size bytes, so its results equal that call's bit
 * for bit; a shape whose split needs more scratch than the array holds is rejected
 * with SSCAN_ERR_INVALID_ARG before anything runs.  Every call on one GPU shares
 * that GPU's array: calls that overlap in time on one GPU (other streams, other
 * threads) race on it and must be serialized by the caller.
 */
#define SSCAN_NOALLOC_SCRATCH_BYTES (32u << 20)
sscan_status sscan_fwd_noalloc(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                               unsigned int flags, const void* x, const void* delta, const float* A,
                               const void* B, const void* C, const float* D, const void* z,
                               const float* delta_bias, const float* initial_state, void* y,
                               float* last_state, void* stream);

/*
 * One recurrent step for a single token per batch row (decode).
 *
 *   state          : [batch, dim, dstate]  (float32) read, then overwritten in place
 *   x, delta, z, y : [batch, dim]          (dtype)
 *   A              : [dim, dstate]         (float32)
 *   B, C           : [batch, dstate]       (dtype)
 *   D, delta_bias  : [dim]                 (float32)
 *
 * Optional (NULL allowed): D, z, delta_bias.  Equivalent to sscan_fwd with
 * seqlen = 1, initial_state = last_state = state.
 */
sscan_status sscan_step(int64_t batch, int64_t dim, int64_t dstate, int dtype, unsigned int flags,
                        float* state, const void* x, const void* delta, const float* A,
                        const void* B, const void* C, const float* D, const void* z,
                        const float* delta_bias, void* y, void* stream);

/*
 * sscan_fwd with the short convolution that precedes the scan in a Mamba block,
 * fused into the scan's load: the page-3 report's MambaBlock.forward
 * (Mamba_Model_Report.md, section 3) passes the x branch through a causal depthwise
 * conv1d over time (kernel d_conv, padding d_conv - 1, output cropped to the first
 * L steps) and a SiLU before the selective scan:
 *   u[b,l,d] = silu(conv_b[d] + sum_{k<dconv} conv_w[d,k] * xx[b, l - (dconv-1) + k, d])
 * where xx is x preceded along time by conv_state_in (the dconv - 1 raw inputs
 * before the sequence, oldest first; zeros when NULL).  The scan, skip term and gate
 * then use u in place of x.  conv_state_out receives the last dconv - 1 raw inputs
 * (the cache that MambaBlock.step keeps, section 6), so a prefill hands over to
 * sscan_step_conv.
 *
 *   x              : [batch, seqlen, dim]    (dtype) raw inputs of the convolution
 *   conv_w         : [dim, dconv]            (float32) taps, conv_w[:, dconv-1] on the current input
 *   conv_b         : [dim]                   (float32) or NULL
 *   conv_state_in  : [batch, dim, dconv - 1] (float32) or NULL
 *   conv_state_out : [batch, dim, dconv - 1] (float32) or NULL; may be conv_state_in
 *   other arguments: as sscan_fwd.
 * 1 <= dconv <= SSCAN_MAX_DCONV (else SSCAN_ERR_UNSUPPORTED).  The backward pass does
 * not include the convolution: sscan_bwd differentiates the scan with respect to u.
 */
sscan_status sscan_fwd_conv(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int64_t dconv,
                            int dtype, unsigned int flags, const void* x, const float* conv_w,
                            const float* conv_b, const float* conv_state_in, float* conv_state_out,
                            const void* delta, const float* A, const void* B, const void* C,
                            const float* D, const void* z, const float* delta_bias,
                            const float* initial_state, void* y, float* last_state, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * sscan_step with the convolution prologue: the page-3 report's MambaBlock.step
 * (section 6) convolves the cached dconv - 1 raw inputs and the new one, applies
 * SiLU, runs the SSM step on the result, and updates the cache by dropping its
 * oldest entry and appending the new raw input.
 *
 *   conv_state : [batch, dim, dconv - 1] (float32) read, then updated in place
 *                (may be NULL only when dconv == 1)
 *   x          : [batch, dim] (dtype) raw input
 *   conv_w, conv_b, dconv: as sscan_fwd_conv; other arguments: as sscan_step.
 */
sscan_status sscan_step_conv(int64_t batch, int64_t dim, int64_t dstate, int64_t dconv, int dtype,
                             unsigned int flags, float* state, float* conv_state, const void* x,
                             const float* conv_w, const float* conv_b, const void* delta, const float* A,
                             const void* B, const void* C, const float* D, const void* z,
                             const float* delta_bias, void* y, void* stream);

/*
 * Workspace bytes sscan_bwd needs for a shape (0 for an empty problem).  The
 * backward pass cannot run without it: it holds the state checkpoints (one per
 * 8 timesteps), per-channel-tile partial sums of dB and dC, per-batch-row
 * partial sums of dA, dD and ddelta_bias, and the sequence-split buffers of the
 * checkpoint pass.  Contents are scratch: nothing is kept between calls.
 */
size_t sscan_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                int dtype);

/*
 * Backward pass of sscan_fwd: gradients of a scalar loss with respect to every
 * input, given dy = dLoss/dy and, optionally, dlast_state = dLoss/d(last_state).
 *
 * The gradients are the chain rule through the forward definition at the top of
 * this header, run backwards in time: the reverse recurrence
 *   g_l = gyo_l C_l + Abar_{l+1} g_{l+1},   gyo_l = dy_l silu(z_l)   (elementwise in N)
 * that the page-3 report's PScan.backward computes with its reverse scan
 * pscan_rev (Mamba_Model_Report.md, section 4.1), with the forward states
 * recomputed rather than stored (the recomputation that the lengnian.github.io
 * notes, "Part3: Mamba - A Selective SSM", list in the hardware-aware algorithm).
 * Gradients then follow per step (phi = Bbar / B):
 *   dx = gyo D + sum_n g phi B        dB = sum_d g phi x        dC = sum_d gyo h
 *   dz = dy (C.h + D x) silu'(z)      dD = sum_{b,l} gyo x
 *   ddelta = sigmoid(delta + delta_bias) sum_n g (A Abar h_{l-1} + dphi/dDelta B x)
 *   dA = sum_{b,l} g (Delta Abar h_{l-1} + dphi/dA B x),  ddelta_bias = sum_{b,l} ddelta
 *   dinitial_state = Abar_0 g_0
 * (zero-order hold: phi = (Abar - 1)/A, dphi/dDelta = Abar, dphi/dA = (Delta Abar - phi)/A,
 * Delta^2/2 at A = 0; SSCAN_FLAG_EULER: phi = Delta, dphi/dDelta = 1, dphi/dA = 0).
 *
 *   inputs  : as sscan_fwd (x, delta, A, B, C, D, z, delta_bias, initial_state, flags)
 *   dy      : [batch, seqlen, dim]    (dtype)
 *   dlast_state : [batch, dim, dstate] (float32), NULL = zero
 *   dx, ddelta, dz : [batch, seqlen, dim]    (dtype)
 *   dB, dC         : [batch, seqlen, dstate] (dtype)
 *   dA             : [dim, dstate]           (float32)
 *   dD, ddelta_bias: [dim]                   (float32)
 *   dinitial_state : [batch, dim, dstate]    (float32)
 *
 * Required: x, delta, A, B, C, dy, dx, ddelta, dA, dB, dC and the workspace
 * (at least sscan_bwd_workspace_size bytes, 256-byte aligned).  dz is required
 * exactly when z is given; dD may be given only with D; ddelta_bias and
 * dinitial_state are optional whether or not delta_bias / initial_state are
 * (they are then the gradients at a zero bias / zero initial state).
 * Outputs must not overlap inputs, each other or the workspace.  Reductions run
 * in a fixed order: results are bitwise reproducible.
 */
sscan_status sscan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                       unsigned int flags, const void* x, const void* delta, const float* A, const void* B,
                       const void* C, const float* D, const void* z, const float* delta_bias,
                       const float* initial_state, const void* dy, const float* dlast_state, void* dx,
                       void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz,
                       float* ddelta_bias, float* dinitial_state, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * Saved checkpoints for a training step.  The lengnian.github.io notes ("Part3:
 * Mamba - A Selective SSM") list recomputation among the means by which the
 * hardware-aware algorithm keeps intermediate results small; sscan_bwd recomputes
 * the forward states from scratch.  A training step that runs the forward anyway
 * can instead keep the state at a coarse grain: sscan_fwd_checkpointed writes the
 * state entering every block of 8 timesteps (1/8 of the four-dimensional state,
 * nothing in between), and sscan_bwd_checkpointed starts its reverse pass from
 * those states instead of running the forward recurrence again.
 *
 * Layout: checkpoints[b][j][n][d], float32, j = 0 .. ceil(seqlen / 8) - 1, holding
 * h_{8j-1}, the state entering timestep 8j (the initial state for j = 0).
 */

/* Bytes of the checkpoint array for a shape (0 for an empty problem). */
size_t sscan_checkpoint_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);

/*
 * sscan_fwd that also writes the checkpoints.
 *   checkpoints      : written; at least sscan_checkpoint_bytes bytes, 4-byte aligned,
 *                      overlapping no other tensor or the workspace
 *   checkpoint_bytes : its size in bytes
 * Other arguments, results and errors: as sscan_fwd (there is no convolution
 * prologue here: the backward pass does not cover it).  y and last_state equal
 * sscan_fwd's bit for bit.
 */
sscan_status sscan_fwd_checkpointed(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                                    unsigned int flags, const void* x, const void* delta, const float* A,
                                    const void* B, const void* C, const float* D, const void* z,
                                    const float* delta_bias, const float* initial_state, void* y,
                                    float* last_state, void* workspace, size_t workspace_bytes,
                                    float* checkpoints, size_t checkpoint_bytes, void* stream);

/* Workspace bytes sscan_bwd_checkpointed needs: sscan_bwd's less the checkpoint array. */
size_t sscan_bwd_checkpointed_workspace_size(int64_t batch, int64_t seqlen, int64_t dim,
                                             int64_t dstate, int dtype);

/*
 * sscan_bwd from checkpoints that sscan_fwd_checkpointed wrote for the same x,
 * delta, A, B, C, delta_bias, initial_state and flags.  The initial state reaches
 * the backward pass through checkpoint block 0, so it is not an argument here;
 * dinitial_state is still produced.
 *   checkpoints      : read; at least sscan_checkpoint_bytes bytes, 4-byte aligned
 *   workspace        : at least sscan_bwd_checkpointed_workspace_size bytes
 * Other arguments, results and errors: as sscan_bwd.  The gradients equal
 * sscan_bwd's to rounding: sscan_bwd's own recomputation may split the sequence
 * differently from the forward, which rounds the states differently.
 */
sscan_status sscan_bwd_checkpointed(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                                    unsigned int flags, const void* x, const void* delta, const float* A,
                                    const void* B, const void* C, const float* D, const void* z,
                                    const float* delta_bias, const float* checkpoints,
                                    size_t checkpoint_bytes, const void* dy, const float* dlast_state,
                                    void* dx, void* ddelta, float* dA, void* dB, void* dC, float* dD,
                                    void* dz, float* ddelta_bias, float* dinitial_state, void* workspace,
                                    size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SELSCAN_H */

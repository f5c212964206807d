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
 *    stream).  The library allocates no device memory and never synchronizes.
 *  - Errors: a nonzero sscan_status is returned and nothing is launched;
 *    sscan_last_error() gives a message (per calling thread).  Arguments are
 *    checked on the host before any launch.  Values are not checked: NaN and
 *    Inf propagate.  SSCAN_ERR_HIP reports a failed launch.
 *  - Outputs must not overlap inputs, except where stated (in-place state).
 *  - dstate (N) must be in [1, SSCAN_MAX_DSTATE].
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

#define SSCAN_VERSION 200
#define SSCAN_MAX_DSTATE 16

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
 * one), which is slower but equally correct.
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
int sscan_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
              unsigned int flags, const void* x, const void* delta, const float* A, const void* B, const void* C,
              const float* D, const void* z, const float* delta_bias,
              const float* initial_state, void* y, float* last_state,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Same as sscan_fwd, with the number of sequence segments chosen by the caller
 * (num_segments >= 1; it is clamped to what the workspace and seqlen allow).
 * num_segments == 0 means "choose automatically" and equals sscan_fwd.
 * For tuning and testing the two-level split; results agree with sscan_fwd
 * up to float32 rounding.
 */
int sscan_fwd_segmented(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                        unsigned int flags, const void* x, const void* delta, const float* A, const void* B,
                        const void* C, const float* D, const void* z, const float* delta_bias,
                        const float* initial_state, void* y, float* last_state,
                        void* workspace, size_t workspace_bytes, int64_t num_segments,
                        void* stream);

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
int sscan_step(int64_t batch, int64_t dim, int64_t dstate, int dtype, unsigned int flags,
               float* state, const void* x, const void* delta, const float* A,
               const void* B, const void* C, const float* D, const void* z,
               const float* delta_bias, void* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SELSCAN_H */

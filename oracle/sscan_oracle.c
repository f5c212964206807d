/*
 * Oracle for the selective state-space scan: a plain, sequential fp64 CPU
 * implementation.  TEST INFRASTRUCTURE ONLY -- it exists to check the HIP
 * library, never to serve results in its place.  It shares no code, header,
 * table or helper with the GPU path.
 *
 * What it computes (per batch row b and channel d, state vector h of length N):
 *
 *   v      = dt[b,l,d] + bias[d]                       (bias = 0 when absent)
 *   Delta  = softplus(v) = log(1 + exp(v))
 *   for each state n:
 *     a      = Delta * A[d,n]
 *     Abar   = exp(a)                                  zero-order hold, diagonal A
 *     Bbar   = (exp(a) - 1) / A[d,n] * B[b,l,n]       = (Delta A)^-1 (exp(Delta A) - 1) Delta B
 *              (Delta * B[b,l,n] in the limit A[d,n] = 0)
 *     h[n]   = Abar * h[n] + Bbar * x[b,l,d]
 *   y      = sum_n C[b,l,n] * h[n] + Dskip[d] * x[b,l,d]
 *   y     *= z * sigmoid(z)                            (only when z is given)
 *
 * Variant (euler != 0): Bbar = Delta * B[b,l,n], the first-order rule that the
 * page-3 report's code uses (section 4.2, selective_scan_seq: deltaB = delta * B);
 * Abar stays exp(Delta A).
 *
 * Sources (the reference pages):
 *  - ZOH formulas Abar = exp(Delta A), Bbar = (Delta A)^-1 (exp(Delta A) - I) Delta B:
 *    velog.io Mamba paper review, section "2 State Space Models", "Discretization";
 *    the integral form A^-1 (e^{A Delta} - I) B is derived on the fakeeyes2wo.github.io
 *    "mamba 学习" page, section "MAMBA" (zero-order-hold derivation).
 *  - Recurrence h_k = Abar h_{k-1} + Bbar x_k, y_k = C h_k (y sees the state that already
 *    includes x_k): velog.io review, "Discretization" item 3; same indexing as the
 *    sequential loop of the page-3 report (gh.r-mj.com Mamba_Model_Report.md,
 *    section 4.2 "selective_scan 和 selective_scan_seq").
 *  - Input-dependent step: Delta = softplus(parameter + projection), shapes
 *    Delta (B,L,D), A (D,N), B/C (B,L,N): velog.io review, section 3.2
 *    "Improving SSMs with Selection".
 *  - Skip term y += D x and the SiLU gate y * silu(z): page-3 report, sections 3
 *    (MambaBlock.forward) and 4.2 (y = y + D * x).
 *  - Single-token recurrent step on a carried state (B, ED, N): page-3 report,
 *    section 6 (ssm_step).
 *
 * Layouts (all row-major, contiguous, fp64):
 *   x, dt, z, y : [batch][seqlen][dim]
 *   B, C        : [batch][seqlen][dstate]
 *   A           : [dim][dstate]
 *   Dskip, bias : [dim]
 *   h0, h_last  : [batch][dim][dstate]
 *
 * Threads only split the independent (b, d) rows; every row is computed by the
 * same sequential loop, in the same order, whatever the thread count.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <omp.h>

/* softplus(v) = log(1 + e^v), written so that neither branch overflows. */
static double softplus(double v) {
  if (v > 0.0) return v + log1p(exp(-v));
  return log1p(exp(v));
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* One (b, d) row of the forward scan over all seqlen steps. */
static void scan_row(int64_t b, int64_t d, int64_t L, int64_t Dm, int64_t N, int euler,
                     const double* x, const double* dt, const double* A,
                     const double* Bm, const double* Cm, const double* Dskip,
                     const double* z, const double* bias, const double* h0,
                     double* y, double* h_last, double* h /* scratch of N */) {
  for (int64_t n = 0; n < N; ++n) h[n] = h0 ? h0[(b * Dm + d) * N + n] : 0.0;
  const double bd = bias ? bias[d] : 0.0;
  for (int64_t l = 0; l < L; ++l) {
    const int64_t i = (b * L + l) * Dm + d;     /* index into [B,L,D] */
    const int64_t r = (b * L + l) * N;          /* row of B, C at (b,l) */
    const double delta = softplus(dt[i] + bd);
    const double xv = x[i];
    double acc = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double an = A[d * N + n];
      const double a = delta * an;
      const double abar = exp(a);
      const double bbar = (an != 0.0 && !euler) ? expm1(a) / an * Bm[r + n] : delta * Bm[r + n];
      h[n] = abar * h[n] + bbar * xv;
      acc += Cm[r + n] * h[n];
    }
    if (Dskip) acc += Dskip[d] * xv;
    if (z) acc *= silu(z[i]);
    y[i] = acc;
  }
  if (h_last)
    for (int64_t n = 0; n < N; ++n) h_last[(b * Dm + d) * N + n] = h[n];
}

int oracle_nthreads_default(void) { return omp_get_max_threads(); }

/* Forward scan.  h0 may be NULL (zero initial state); h_last may be NULL.
 * euler != 0 selects Bbar = Delta * B.
 * Returns the number of threads used, or -1 on a bad argument. */
int oracle_sscan_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int euler,
                     const double* x, const double* dt, const double* A,
                     const double* Bm, const double* Cm, const double* Dskip,
                     const double* z, const double* bias, const double* h0,
                     double* y, double* h_last, int nthreads) {
  if (batch < 0 || seqlen < 0 || dim < 0 || dstate < 1 || dstate > 4096) return -1;
  if (nthreads < 1) nthreads = omp_get_max_threads();
  const int64_t rows = batch * dim;
  int used = 1;
#pragma omp parallel num_threads(nthreads)
  {
    double h[4096];
#pragma omp single
    used = omp_get_num_threads();
#pragma omp for schedule(dynamic, 1)
    for (int64_t rd = 0; rd < rows; ++rd) {
      const int64_t b = rd / dim, d = rd % dim;
      scan_row(b, d, seqlen, dim, dstate, euler, x, dt, A, Bm, Cm, Dskip, z, bias, h0, y, h_last, h);
    }
  }
  return used;
}

/* One recurrent step: the forward scan with seqlen = 1, starting from and
 * writing back `state` [batch][dim][dstate].  Token tensors are [batch][dim]
 * and [batch][dstate]. */
int oracle_sscan_step(int64_t batch, int64_t dim, int64_t dstate, int euler, double* state,
                      const double* x, const double* dt, const double* A,
                      const double* Bm, const double* Cm, const double* Dskip,
                      const double* z, const double* bias, double* y, int nthreads) {
  if (batch < 0 || dim < 0 || dstate < 1 || dstate > 4096) return -1;
  if (nthreads < 1) nthreads = omp_get_max_threads();
  const int64_t rows = batch * dim;
  int used = 1;
#pragma omp parallel num_threads(nthreads)
  {
    double h[4096];
#pragma omp single
    used = omp_get_num_threads();
#pragma omp for schedule(static)
    for (int64_t rd = 0; rd < rows; ++rd) {
      const int64_t b = rd / dim, d = rd % dim;
      /* seqlen = 1: the [B,1,D] and [B,1,N] layouts coincide with [B,D] and [B,N]. */
      scan_row(b, d, 1, dim, dstate, euler, x, dt, A, Bm, Cm, Dskip, z, bias, state, y, state, h);
    }
  }
  return used;
}

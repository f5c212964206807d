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
#include <stdlib.h>
#include <string.h>
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

/* ---------------------------------------------------------------------------
 * Backward pass (gradients of a scalar loss through the forward scan).
 *
 * Given dy = dLoss/dy [batch][seqlen][dim] and, optionally, dhL = dLoss/d(last
 * state) [batch][dim][dstate], it returns the gradients with respect to every
 * input.  This is the chain rule applied to the forward definition above, run
 * backwards in time (the reverse recurrence the page-3 report's pscan_rev serves,
 * section 4.1):
 *
 *   s(z)    = silu(z), s'(z) = sigmoid(z) (1 + z (1 - sigmoid(z)))
 *   yo_l    = sum_n C[l,n] h_l[n] + D x_l                 (output before the gate)
 *   gyo_l   = dy_l s(z_l)            dz_l = dy_l yo_l s'(z_l)
 *   gh_l[n] = gyo_l C[l,n] + Abar_{l+1}[n] gh_{l+1}[n]     (gh_{L-1} also gets dhL)
 *   dC[l,n] = sum_d gyo_l h_l[n]
 *   dx_l    = gyo_l D + sum_n gh_l[n] phi_l[n] B[l,n]      phi = Bbar / B
 *   dB[l,n] = sum_d gh_l[n] phi_l[n] x_l
 *   dDelta  = sum_n gh_l[n] (A[n] Abar h_{l-1}[n] + dphi/dDelta B[l,n] x_l)
 *   dA[n]   = sum_{b,l} gh_l[n] (Delta Abar h_{l-1}[n] + dphi/dA B[l,n] x_l)
 *   ddt     = dDelta sigmoid(dt + bias);   dbias = sum_{b,l} ddt;   dD = sum_{b,l} gyo x
 *   dh0[n]  = Abar_0[n] gh_0[n]
 *
 * with, for the zero-order hold, phi = (exp(Delta A) - 1)/A, dphi/dDelta = Abar,
 * dphi/dA = (Delta Abar - phi)/A (Delta^2/2 at A = 0); for the Euler rule phi =
 * Delta, dphi/dDelta = 1, dphi/dA = 0.  dphi/dA is evaluated as
 * Delta^2 * (u e^u - e^u + 1)/u^2 with u = Delta A, and that ratio by its Taylor
 * series sum_k (k+1) u^k/(k+2)! when |u| < 0.5 (where the closed form cancels).
 * --------------------------------------------------------------------------- */

static double sigmoid(double v) {
  if (v >= 0.0) return 1.0 / (1.0 + exp(-v));
  const double e = exp(v);
  return e / (1.0 + e);
}

/* (u e^u - e^u + 1) / u^2, i.e. d/du of expm1(u)/u. */
static double dphi1(double u) {
  if (fabs(u) < 0.5) {
    double term = 0.5, sum = 0.0;          /* (k+1) u^k / (k+2)!, k = 0, 1, ... */
    double uk = 1.0, fact = 2.0;           /* u^k and (k+2)! */
    for (int k = 0; k < 30; ++k) {
      term = (k + 1) * uk / fact;
      sum += term;
      uk *= u;
      fact *= (double)(k + 3);
      if (fabs(term) < 1e-18 * fabs(sum)) break;
    }
    return sum;
  }
  return (u * exp(u) - expm1(u)) / (u * u);
}

/* One batch row b, all channels: forward with stored states, then the reverse
 * pass.  dB, dC rows of this b are owned by the caller's thread; dA, dD, dbias
 * contributions go to this row's partial arrays pA [dim][N], pD [dim], pb [dim]. */
static void bwd_row(int64_t b, int64_t L, int64_t Dm, int64_t N, int euler,
                    const double* x, const double* dt, const double* A, const double* Bm,
                    const double* Cm, const double* Dskip, const double* z, const double* bias,
                    const double* h0, const double* dy, const double* dhL,
                    double* dx, double* ddt, double* dBm, double* dCm, double* dz, double* dh0,
                    double* pA, double* pD, double* pb,
                    double* hs /* (L+1) N */, double* ab /* L N */, double* gh /* N */) {
  for (int64_t l = 0; l < L; ++l)
    for (int64_t n = 0; n < N; ++n) {
      dBm[(b * L + l) * N + n] = 0.0;
      dCm[(b * L + l) * N + n] = 0.0;
    }
  for (int64_t d = 0; d < Dm; ++d) {
    const double bd = bias ? bias[d] : 0.0;
    /* forward, keeping every state: hs[l*N + n] is the state before step l */
    for (int64_t n = 0; n < N; ++n) hs[n] = h0 ? h0[(b * Dm + d) * N + n] : 0.0;
    for (int64_t l = 0; l < L; ++l) {
      const int64_t i = (b * L + l) * Dm + d, r = (b * L + l) * N;
      const double delta = softplus(dt[i] + bd);
      for (int64_t n = 0; n < N; ++n) {
        const double an = A[d * N + n];
        const double abar = exp(delta * an);
        const double phi = (an != 0.0 && !euler) ? expm1(delta * an) / an : delta;
        ab[l * N + n] = abar;
        hs[(l + 1) * N + n] = abar * hs[l * N + n] + phi * Bm[r + n] * x[i];
      }
    }
    /* reverse */
    for (int64_t n = 0; n < N; ++n) gh[n] = dhL ? dhL[(b * Dm + d) * N + n] : 0.0;  /* Abar_{l+1} gh_{l+1} */
    for (int64_t l = L - 1; l >= 0; --l) {
      const int64_t i = (b * L + l) * Dm + d, r = (b * L + l) * N;
      const double v = dt[i] + bd;
      const double delta = softplus(v);
      const double xv = x[i];
      double yo = 0.0;
      for (int64_t n = 0; n < N; ++n) yo += Cm[r + n] * hs[(l + 1) * N + n];
      if (Dskip) yo += Dskip[d] * xv;
      double gyo = dy[i];
      if (z) {
        const double zz = z[i], sg = sigmoid(zz);
        gyo = dy[i] * zz * sg;
        dz[i] = dy[i] * yo * sg * (1.0 + zz * (1.0 - sg));
      }
      double gx = Dskip ? gyo * Dskip[d] : 0.0;
      double gdelta = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        const double an = A[d * N + n];
        const double abar = ab[l * N + n];
        const double hprev = hs[l * N + n];
        const double g = gyo * Cm[r + n] + gh[n];   /* gh_l */
        const int zoh = (an != 0.0 && !euler);
        const double phi = zoh ? expm1(delta * an) / an : delta;
        const double dphi_ddelta = euler ? 1.0 : abar;
        const double dphi_dA = euler ? 0.0 : delta * delta * dphi1(delta * an);
        dCm[r + n] += gyo * hs[(l + 1) * N + n];
        dBm[r + n] += g * phi * xv;
        gx += g * phi * Bm[r + n];
        gdelta += g * (an * abar * hprev + dphi_ddelta * Bm[r + n] * xv);
        pA[d * N + n] += g * (delta * abar * hprev + dphi_dA * Bm[r + n] * xv);
        gh[n] = abar * g;
      }
      dx[i] = gx;
      const double gdt = gdelta * sigmoid(v);
      ddt[i] = gdt;
      pb[d] += gdt;
      if (Dskip) pD[d] += gyo * xv;
    }
    if (dh0)
      for (int64_t n = 0; n < N; ++n) dh0[(b * Dm + d) * N + n] = gh[n];
  }
}

/* Backward pass.  Required: x, dt, A, Bm, Cm, dy and the outputs dx, ddt, dA, dB, dC.
 * Optional inputs Dskip, z, bias, h0, dhL (NULL = absent / zero); optional outputs
 * dD (needs Dskip), dz (needs z), dbias, dh0.  Returns threads used or -1. */
int oracle_sscan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int euler,
                     const double* x, const double* dt, const double* A, const double* Bm,
                     const double* Cm, const double* Dskip, const double* z, const double* bias,
                     const double* h0, const double* dy, const double* dhL,
                     double* dx, double* ddt, double* dA, double* dB, double* dC, double* dD,
                     double* dz, double* dbias, double* dh0, int nthreads) {
  if (batch < 0 || seqlen < 0 || dim < 0 || dstate < 1 || dstate > 4096) return -1;
  if ((z == NULL) != (dz == NULL) && dz != NULL) return -1;
  if (nthreads < 1) nthreads = omp_get_max_threads();
  const int64_t N = dstate;
  double* pA = (double*)calloc((size_t)(batch > 0 ? batch : 1) * dim * N + 1, sizeof(double));
  double* pD = (double*)calloc((size_t)(batch > 0 ? batch : 1) * dim + 1, sizeof(double));
  double* pb = (double*)calloc((size_t)(batch > 0 ? batch : 1) * dim + 1, sizeof(double));
  if (!pA || !pD || !pb) { free(pA); free(pD); free(pb); return -1; }
  double* dz_use = z ? dz : NULL;
  int used = 1;
  int fail = 0;
#pragma omp parallel num_threads(nthreads)
  {
    double* hs = (double*)malloc((size_t)(seqlen + 1) * N * sizeof(double));
    double* ab = (double*)malloc((size_t)(seqlen > 0 ? seqlen : 1) * N * sizeof(double));
    double* gh = (double*)malloc((size_t)N * sizeof(double));
#pragma omp single
    used = omp_get_num_threads();
    if (!hs || !ab || !gh) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t b = 0; b < batch; ++b) {
      if (hs && ab && gh)
        bwd_row(b, seqlen, dim, N, euler, x, dt, A, Bm, Cm, Dskip, z, bias, h0, dy, dhL, dx, ddt, dB, dC,
                dz_use, dh0, pA + b * dim * N, pD + b * dim, pb + b * dim, hs, ab, gh);
    }
    free(hs);
    free(ab);
    free(gh);
  }
  if (!fail) {
    /* batch rows summed in a fixed order */
    for (int64_t k = 0; k < dim * N; ++k) {
      double s = 0.0;
      for (int64_t b = 0; b < batch; ++b) s += pA[b * dim * N + k];
      dA[k] = s;
    }
    for (int64_t d = 0; d < dim; ++d) {
      double sD = 0.0, sb = 0.0;
      for (int64_t b = 0; b < batch; ++b) {
        sD += pD[b * dim + d];
        sb += pb[b * dim + d];
      }
      if (dD) dD[d] = Dskip ? sD : 0.0;
      if (dbias) dbias[d] = sb;
    }
  }
  free(pA);
  free(pD);
  free(pb);
  return fail ? -1 : used;
}

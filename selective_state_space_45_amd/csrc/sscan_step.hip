// One recurrent step of the selective scan (decode), gfx950.
//
// Computes, for a single token per batch row (page-3 report, section 6, ssm_step;
// discretization as in the velog.io review, "Discretization"):
//   Delta = softplus(dt + bias), Abar = exp(Delta A), Bbar = (Abar - 1)/A * B
//   (Delta * B when A == 0), h <- Abar h + Bbar x (in place), y = (C . h + D x) silu(z).
//
// The step is bound by reading and writing the fp32 state [batch, dim, N].
// LPR lanes share one (b, d) row and each holds 4 consecutive states, so the
// state is read and written with fully coalesced 16-byte accesses; the partial
// C . h of the row is summed across its lanes with cross-lane shuffles.
#include "sscan_device.h"
#include "sscan_internal.h"

namespace sscan {

template <typename Tin, int LPR, bool VEC>
__global__ __launch_bounds__(256) void step_kernel(StepParams p) {
  const Tin* __restrict__ X = static_cast<const Tin*>(p.x);
  const Tin* __restrict__ DT = static_cast<const Tin*>(p.dt);
  const Tin* __restrict__ Z = static_cast<const Tin*>(p.z);
  const Tin* __restrict__ Bp = static_cast<const Tin*>(p.B);
  const Tin* __restrict__ Cp = static_cast<const Tin*>(p.C);
  Tin* __restrict__ Y = static_cast<Tin*>(p.y);
  float* __restrict__ S = p.state;

  const int64_t rows = p.batch * p.dim;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t row = gid / LPR;
  const int q = static_cast<int>(gid - row * LPR);
  const bool rvalid = row < rows;
  const int64_t rr = rvalid ? row : 0;
  const int64_t b = rr / p.dim, d = rr - b * p.dim;
  const int N = p.N;
  const int n0 = 4 * q;

  float yp = 0.f, xv = 0.f;
  if (rvalid) {
    xv = to_f32(X[rr]);
    const float v2 = fmaf(to_f32(DT[rr]), kLog2e, p.bias ? p.bias[d] * kLog2e : 0.f);
    const float d2 = softplus_log2e(v2);  // Delta * log2(e)
    const float* Ad = p.A + d * N + n0;
    float* Sd = S + rr * N + n0;
    const Tin* Bb = Bp + b * N + n0;
    const Tin* Cb = Cp + b * N + n0;
    float h[4] = {0.f, 0.f, 0.f, 0.f}, a[4] = {0.f, 0.f, 0.f, 0.f};
    if (VEC && n0 < N) {
      const float4 hv = *reinterpret_cast<const float4*>(Sd);
      const float4 av = *reinterpret_cast<const float4*>(Ad);
      h[0] = hv.x; h[1] = hv.y; h[2] = hv.z; h[3] = hv.w;
      a[0] = av.x; a[1] = av.y; a[2] = av.z; a[3] = av.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (n0 + j < N) { h[j] = Sd[j]; a[j] = Ad[j]; }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (n0 + j < N) {
        const float e = hw_exp2(d2 * a[j]);
        const float g = (a[j] != 0.f) ? (e - 1.f) / a[j] : d2 * kLn2;
        h[j] = fmaf(e, h[j], g * to_f32(Bb[j]) * xv);
        yp = fmaf(to_f32(Cb[j]), h[j], yp);
      }
    }
    if (VEC && n0 < N) {
      *reinterpret_cast<float4*>(Sd) = make_float4(h[0], h[1], h[2], h[3]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (n0 + j < N) Sd[j] = h[j];
    }
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) yp += __shfl_xor(yp, off);
  if (rvalid && q == 0) {
    float yv = yp + (p.Dskip ? p.Dskip[d] * xv : 0.f);
    if (Z) yv *= silu(to_f32(Z[rr]));
    store_val(&Y[rr], yv);
  }
}

hipError_t launch_step(const StepParams& p, bool bf16, hipStream_t s) {
  const int64_t rows = p.batch * p.dim;
  if (rows <= 0) return hipSuccess;
  const int lpr = (p.N <= 4) ? 1 : (p.N <= 8 ? 2 : 4);
  const bool vec = (p.N % 4 == 0) && ((reinterpret_cast<uintptr_t>(p.state) & 15) == 0) &&
                   ((reinterpret_cast<uintptr_t>(p.A) & 15) == 0);
  const int64_t threads = rows * lpr;
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256)), block(256);
#define SSCAN_STEP(TIN, LP, V) hipLaunchKernelGGL((step_kernel<TIN, LP, V>), grid, block, 0, s, p)
#define SSCAN_STEP_LPR(TIN, V)       \
  switch (lpr) {                     \
    case 1: SSCAN_STEP(TIN, 1, V); break; \
    case 2: SSCAN_STEP(TIN, 2, V); break; \
    default: SSCAN_STEP(TIN, 4, V); break; \
  }
  if (bf16) {
    if (vec) { SSCAN_STEP_LPR(bf16_t, true) } else { SSCAN_STEP_LPR(bf16_t, false) }
  } else {
    if (vec) { SSCAN_STEP_LPR(float, true) } else { SSCAN_STEP_LPR(float, false) }
  }
#undef SSCAN_STEP_LPR
#undef SSCAN_STEP
  return hipGetLastError();
}

}  // namespace sscan

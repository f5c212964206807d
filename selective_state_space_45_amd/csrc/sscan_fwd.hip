// Forward selective scan: segment carry and fill kernels, and the dispatch of the
// scan launches to the (mode, discretization rule) variants compiled in
// sscan_fwd_zoh.hip, sscan_fwd_euler.hip (one or two states per wave) and
// sscan_fwd_row_zoh.hip, sscan_fwd_row_euler.hip (states across the lanes of a row).
#include "sscan_fwd_kernel.h"
#include "sscan_fwd_row.h"

namespace sscan {

extern template hipError_t launch_fwd_variant<kFwdOut, false, false>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_fwd_variant<kFwdAgg, false, false>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_fwd_variant<kFwdOut, true, false>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_fwd_variant<kFwdAgg, true, false>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_fwd_variant<kFwdOutCkpt, false, false>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_fwd_variant<kFwdOutCkpt, true, false>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_fwd_variant<kFwdOut, false, true>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_fwd_variant<kFwdAgg, false, true>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_fwd_variant<kFwdOut, true, true>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_fwd_variant<kFwdAgg, true, true>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_fwd_row<kFwdOut, false>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_fwd_row<kFwdCkpt, false>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_fwd_row<kFwdOutCkpt, false>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_fwd_row<kFwdOut, true>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_fwd_row<kFwdCkpt, true>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_fwd_row<kFwdOutCkpt, true>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_fwd_row<kFwdOutConv, false>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_fwd_row<kFwdOutConv, true>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_fwd_row<kFwdOut, false, true>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_fwd_row<kFwdCkptAgg, false>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_fwd_row<kFwdCkptAgg, true>(const FwdParams&, bool, hipStream_t);

// carry[s] = state entering segment s: carry[0] = h_init (or 0),
// carry[s+1] = exp2(A * S_s) * carry[s] + hend_s, where S_s is the segment's sum of
// Delta*log2(e), so exp2(A * S_s) is the product of Abar over the segment.
__global__ __launch_bounds__(256) void carry_kernel(const float* __restrict__ agg_h, const float* __restrict__ agg_s,
                                                    const float* __restrict__ A, const float* __restrict__ h_init,
                                                    float* __restrict__ carry, int64_t batch, int64_t dim, int N,
                                                    int nseg) {
  const int64_t total = batch * dim * N;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t bd = i / N;
  const int n = static_cast<int>(i - bd * N);
  const int64_t d = bd % dim;
  const float a = A[d * N + n];
  float c = h_init ? h_init[i] : 0.f;
  // Segments in groups of G: the group's aggregates are loaded together, so their
  // latencies overlap instead of adding up along the sequential combine (one round
  // of loads for up to 16 segments).
  constexpr int G = 16;
  for (int s0 = 0; s0 < nseg; s0 += G) {
    float hv[G], sv[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int s = s0 + k;
      const bool have = s + 1 < nseg;   // the last segment has no aggregate
      hv[k] = have ? agg_h[static_cast<int64_t>(s) * total + i] : 0.f;
      sv[k] = have ? agg_s[static_cast<int64_t>(s) * batch * dim + bd] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int s = s0 + k;
      if (s < nseg) {
        carry[static_cast<int64_t>(s) * total + i] = c;
        c = fmaf(hw_exp2(a * sv[k]), c, hv[k]);
      }
    }
  }
}

__global__ __launch_bounds__(256) void fill_state_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                                         int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.f;
}

// Launches taken by the row layout (fwd_row_kernel): N <= 16 and one workgroup per CU
// at a time (the one-state-per-wave grids), with or without the convolution
// prologue.  Measured on the training shape (batch 8, seqlen 4096, dim 2048, N 16,
// bf16), steady state: 0.40 ms against 0.45 for fwd_kernel with one state per wave;
// Euler rule 0.35 against 0.43; with a 4-tap convolution prologue 0.48 against 0.58.
bool fwd_row_layout(const FwdParams& p) { return p.N <= 16 && p.npw == 1; }

// Waves per workgroup: N / (states per wave) rounded up to a power of two (at most 16).
int fwd_nsplit(int npw, int N) {
  const int per = (npw == 2 && N >= 3) ? 2 : 1;
  const int need = (N + per - 1) / per;
  int ns = 1;
  while (ns < need) ns <<= 1;
  return ns;
}

namespace {

template <int MODE>
hipError_t launch_fwd_mode(const FwdParams& p, bool bf16, hipStream_t s) {
  if constexpr (MODE == kFwdOut || MODE == kFwdAgg) {   // the modes with a convolution prologue
    if (p.conv_w) {
      if constexpr (MODE == kFwdOut) {
        if (fwd_row_layout(p))
          return p.euler ? launch_fwd_row<kFwdOutConv, true>(p, bf16, s)
                         : launch_fwd_row<kFwdOutConv, false>(p, bf16, s);
      }
      return p.euler ? launch_fwd_variant<MODE, true, true>(p, bf16, s)
                     : launch_fwd_variant<MODE, false, true>(p, bf16, s);
    }
  }
  if constexpr (MODE == kFwdOut) {
    // a rank-one A stated by the caller: the row layout's factored staging (it checks
    // the form per workgroup and falls back to the plain staging where it fails)
    if (p.structured && !p.euler && fwd_row_layout(p)) return launch_fwd_row<kFwdOut, false, true>(p, bf16, s);
  }
  if constexpr (MODE != kFwdAgg) {
    // the checkpoint pass always runs one state per wave, hence the row layout
    if (MODE == kFwdCkpt || fwd_row_layout(p))
      return p.euler ? launch_fwd_row<MODE, true>(p, bf16, s) : launch_fwd_row<MODE, false>(p, bf16, s);
  }
  if constexpr (MODE != kFwdCkpt)
    return p.euler ? launch_fwd_variant<MODE, true, false>(p, bf16, s) : launch_fwd_variant<MODE, false, false>(p, bf16, s);
  return hipErrorInvalidValue;
}

// out[b][d][k] = raw input at position L - (dconv-1) + k (from x, or from the incoming
// state for positions below 0).  One thread per (b, d): all reads before any write,
// so out may be the same buffer as in.
template <typename Tin>
__global__ __launch_bounds__(256) void conv_state_kernel(const Tin* __restrict__ x, const float* in, float* out,
                                                         int64_t batch, int64_t L, int64_t dim, int dconv) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= batch * dim) return;
  const int64_t b = i / dim, d = i - b * dim;
  const int km = dconv - 1;
  float v[kMaxConv];
#pragma unroll
  for (int k = 0; k < kMaxConv - 1; ++k) {
    v[k] = 0.f;
    if (k < km) {
      const int64_t pos = L - km + k;
      if (pos >= 0)
        v[k] = to_f32(x[(b * L + pos) * dim + d]);
      else if (in)
        v[k] = in[i * km + km + pos];
    }
  }
#pragma unroll
  for (int k = 0; k < kMaxConv - 1; ++k)
    if (k < km) out[i * km + k] = v[k];
}

}  // namespace

hipError_t launch_fwd_main(const FwdParams& p, bool bf16, hipStream_t s) {
  // with a checkpoint array (and no convolution prologue) the output pass saves the
  // backward pass's checkpoints as it goes
  if (p.ckpt && !p.conv_w) return launch_fwd_mode<kFwdOutCkpt>(p, bf16, s);
  return launch_fwd_mode<kFwdOut>(p, bf16, s);
}

hipError_t launch_fwd_aggregate(const FwdParams& p, bool bf16, hipStream_t s) {
  return launch_fwd_mode<kFwdAgg>(p, bf16, s);
}

hipError_t launch_fwd_checkpoints(const FwdParams& p, bool bf16, hipStream_t s) {
  return launch_fwd_mode<kFwdCkpt>(p, bf16, s);
}

hipError_t launch_fwd_checkpoints_agg(const FwdParams& p, bool bf16, hipStream_t s) {
  return p.euler ? launch_fwd_row<kFwdCkptAgg, true>(p, bf16, s) : launch_fwd_row<kFwdCkptAgg, false>(p, bf16, s);
}

hipError_t launch_fwd_carry(const float* agg_h, const float* agg_s, const float* A, const float* h_init, float* carry,
                            int64_t batch, int64_t dim, int N, int nseg, hipStream_t s) {
  const int64_t total = batch * dim * N;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(carry_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s, agg_h, agg_s, A,
                     h_init, carry, batch, dim, N, nseg);
  return hipGetLastError();
}

hipError_t launch_conv_state(const void* x, const float* in, float* out, int64_t batch, int64_t L, int64_t dim,
                             int dconv, bool bf16, hipStream_t s) {
  const int64_t n = batch * dim;
  if (n <= 0 || dconv <= 1) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((n + 255) / 256));
  if (bf16)
    hipLaunchKernelGGL(conv_state_kernel<bf16_t>, grid, dim3(256), 0, s, static_cast<const bf16_t*>(x), in, out, batch, L,
                       dim, dconv);
  else
    hipLaunchKernelGGL(conv_state_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(x), in, out, batch, L,
                       dim, dconv);
  return hipGetLastError();
}

hipError_t launch_fill_state(float* dst, const float* src, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_state_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, dst, src, n);
  return hipGetLastError();
}

}  // namespace sscan

// One recurrent step of the selective scan (decode), gfx950.
//
// Computes, for a single token per batch row (page-3 report, section 6, ssm_step;
// discretization as in the velog.io review, "Discretization"):
//   Delta = softplus(dt + bias), Abar = exp(Delta A), Bbar = (Abar - 1)/A * B
//   (Delta * B when A == 0), h <- Abar h + Bbar x (in place), y = (C . h + D x) silu(z).
// With the Euler rule (page-3 report, section 4.2) Bbar = Delta * B.
// With the convolution prologue (page-3 report, section 6, MambaBlock.step), x is a
// raw input: the scan runs on silu(conv_b + sum_k w[k] window[k]) over the window of
// the dconv - 1 cached raw inputs and x, and the cache drops its oldest entry and
// appends x.
//
// The step is bound by reading and writing the fp32 state [batch, dim, N].  Each
// lane holds 4 or 8 consecutive states of one (b, d) row, read and written with
// 16-byte accesses; the partial C . h of a row is summed across its lanes with
// cross-lane shuffles.
#include "sscan_device.h"
#include "sscan_internal.h"

namespace sscan {

typedef float f32x4v __attribute__((ext_vector_type(4)));

// The state streams through once per step: its loads and stores are marked
// non-temporal (measured on 5 rotating 84 MB states, an in-place float4 update ran at
// 5.5 TB/s with non-temporal accesses against 5.0 TB/s without).
__device__ __forceinline__ float4 load_state4(const float* p) {
  const f32x4v v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_state4(float* p, float a, float b, float c, float d) {
  const f32x4v v = {a, b, c, d};
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4v*>(p));
}

// Four consecutive B or C values of one batch row.
template <typename Tin, bool V>
__device__ __forceinline__ void load4(const Tin* __restrict__ p, int n0, int N, float* v) {
  if constexpr (V && sizeof(Tin) == 2) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(w.x << 16);
    v[1] = __uint_as_float(w.x & 0xffff0000u);
    v[2] = __uint_as_float(w.y << 16);
    v[3] = __uint_as_float(w.y & 0xffff0000u);
  } else if constexpr (V) {
    const float4 f = *reinterpret_cast<const float4*>(p);
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = (n0 + j < N) ? to_f32(p[j]) : 0.f;
  }
}

// SPL states per lane (4 or 8), LPR = ceil(N / SPL) lanes per (b, d) row.  VEC: N is a
// multiple of 4 and state, A, B, C allow 16-byte (8-byte for bf16 B/C) accesses.
// NFIX: N as a compile-time constant (0 = run time).  EULER: Bbar = Delta B.
// CONV: convolution prologue with cache cst [rows][dconv-1], taps cw [dim][dconv].
template <typename Tin, int SPL, int LPR, bool VEC, int NFIX, bool EULER, bool CONV>
__global__ __launch_bounds__(256) void step_kernel(float* __restrict__ S, const Tin* __restrict__ X,
                                                   const Tin* __restrict__ DT, const Tin* __restrict__ Z,
                                                   const Tin* __restrict__ Bp, const Tin* __restrict__ Cp,
                                                   const float* __restrict__ Ag, const float* __restrict__ Dg,
                                                   const float* __restrict__ biasg, Tin* __restrict__ Y, int64_t rows,
                                                   int64_t dim, int Nrt, float* __restrict__ cst,
                                                   const float* __restrict__ cw, const float* __restrict__ cb, int K) {
  const int N = NFIX > 0 ? NFIX : Nrt;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t row = gid / LPR;
  const int q = static_cast<int>(gid - row * LPR);
  if (row >= rows) return;  // whole rows leave together: LPR divides the wave size
  const int64_t b = row / dim, d = row - b * dim;
  const int n0 = SPL * q;

  float yp = 0.f;
  float xv = to_f32(X[row]);
  if constexpr (CONV) {
    // window: cached raw inputs (oldest first) then x; read before any lane updates it
    float* cs = cst + row * (K - 1);
    float win[kMaxConv];
#pragma unroll
    for (int k = 0; k < kMaxConv; ++k) win[k] = (k < K - 1) ? cs[k] : 0.f;
    float acc = cb ? cb[d] : 0.f;
#pragma unroll
    for (int k = 0; k < kMaxConv; ++k) {
      const float v = (k < K - 1) ? win[k] : xv;
      if (k < K) acc = fmaf(cw[d * K + k], v, acc);
    }
    if (q == 0) {
#pragma unroll
      for (int k = 0; k < kMaxConv - 1; ++k)
        if (k < K - 1) cs[k] = (k + 1 < K - 1) ? win[k + 1] : xv;
    }
    xv = silu(acc);
  }
  if (n0 < N) {
    const float v2 = fmaf(to_f32(DT[row]), kLog2e, biasg ? biasg[d] * kLog2e : 0.f);
    float h[SPL], a[SPL], bv[SPL], cv[SPL];
    float* Sd = S + row * N + n0;
    const float* Ad = Ag + d * N + n0;
#pragma unroll
    for (int k = 0; k < SPL / 4; ++k) {
      if constexpr (VEC) {
        // N is a multiple of 4, so a group of 4 states lies wholly inside the row or
        // wholly past it (N = 12: the second lane's upper group); a group past the row
        // is neither read nor written, and contributes zero to C . h
        if (NFIX > 0 || n0 + 4 * k < N) {
          const float4 hv = load_state4(Sd + 4 * k);
          const float4 av = *reinterpret_cast<const float4*>(Ad + 4 * k);
          h[4 * k] = hv.x; h[4 * k + 1] = hv.y; h[4 * k + 2] = hv.z; h[4 * k + 3] = hv.w;
          a[4 * k] = av.x; a[4 * k + 1] = av.y; a[4 * k + 2] = av.z; a[4 * k + 3] = av.w;
          load4<Tin, VEC>(Bp + b * N + n0 + 4 * k, n0 + 4 * k, N, bv + 4 * k);
          load4<Tin, VEC>(Cp + b * N + n0 + 4 * k, n0 + 4 * k, N, cv + 4 * k);
        } else {
#pragma unroll
          for (int j = 4 * k; j < 4 * k + 4; ++j) h[j] = a[j] = bv[j] = cv[j] = 0.f;
        }
      } else {
#pragma unroll
        for (int j = 4 * k; j < 4 * k + 4; ++j) {
          h[j] = (n0 + j < N) ? Sd[j] : 0.f;
          a[j] = (n0 + j < N) ? Ad[j] : 0.f;
        }
        load4<Tin, VEC>(Bp + b * N + n0 + 4 * k, n0 + 4 * k, N, bv + 4 * k);
        load4<Tin, VEC>(Cp + b * N + n0 + 4 * k, n0 + 4 * k, N, cv + 4 * k);
      }
    }
    const float d2 = softplus_log2e(v2);  // Delta * log2(e)
    const float dl = d2 * kLn2;           // Delta
    bool small = false;
#pragma unroll
    for (int j = 0; j < SPL; ++j) small = small || fabsf(a[j]) < kSmallA;
    // (Abar - 1) / A: the accurate zoh_phi where a wave holds some |A| < kSmallA (A = 0
    // included; wave-uniform choice), else the direct quotient
    auto update = [&](auto accurate) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        const float arg = d2 * a[j];
        const float e = hw_exp2(arg);
        const float rA = a[j] != 0.f ? hw_rcp(a[j]) : 0.f;
        const float g = EULER ? dl : (decltype(accurate)::value ? zoh_phi(e, arg, d2, rA) : (e - 1.f) * rA);
        h[j] = fmaf(e, h[j], g * bv[j] * xv);
        yp = fmaf(cv[j], h[j], yp);
      }
    };
    if (EULER || !__any(small))
      update(std::false_type{});
    else
      update(std::true_type{});
#pragma unroll
    for (int k = 0; k < SPL / 4; ++k) {
      if constexpr (VEC) {
        if (NFIX > 0 || n0 + 4 * k < N)
          store_state4(Sd + 4 * k, h[4 * k], h[4 * k + 1], h[4 * k + 2], h[4 * k + 3]);
      } else {
#pragma unroll
        for (int j = 4 * k; j < 4 * k + 4; ++j)
          if (n0 + j < N) Sd[j] = h[j];
      }
    }
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) yp += __shfl_xor(yp, off);
  if (q == 0) {
    float yv = yp + (Dg ? Dg[d] * xv : 0.f);
    if (Z) yv *= silu(to_f32(Z[row]));
    store_val(&Y[row], yv);
  }
}

// The decode step for N = 16 with vector-aligned tensors and no convolution prologue:
// 4 lanes per (b, d) row and 4 states per lane, as step_kernel<.., 4, 4, true, 16, ..>,
// but each thread walks KB batch rows of one channel, so A[d] (and 1/A) is loaded once
// per KB rows instead of once per row: with A read per row, every step moved the whole
// [D, N] A (327 KB at dim 5120) through L2 once per batch row, as much traffic as the
// state itself.  The KB state quads are loaded before any is used.
template <typename Tin, bool EULER, int KB>
__global__ __launch_bounds__(256) void step16_kernel(float* __restrict__ S, const Tin* __restrict__ X,
                                                     const Tin* __restrict__ DT, const Tin* __restrict__ Z,
                                                     const Tin* __restrict__ Bp, const Tin* __restrict__ Cp,
                                                     const float* __restrict__ Ag, const float* __restrict__ Dg,
                                                     const float* __restrict__ biasg, Tin* __restrict__ Y,
                                                     int64_t groups, int64_t dim) {
  constexpr int N = 16;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t rg = gid >> 2;               // (batch group, channel)
  const int q = static_cast<int>(gid & 3);   // lane of the row: states 4q .. 4q + 3
  if (rg >= groups * dim) return;            // whole rows leave together
  const int64_t bg = rg / dim, d = rg - bg * dim;
  const int n0 = 4 * q;

  const float4 av = *reinterpret_cast<const float4*>(Ag + d * N + n0);
  const float a[4] = {av.x, av.y, av.z, av.w};
  float rA[4];
  bool small = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    rA[j] = a[j] != 0.f ? hw_rcp(a[j]) : 0.f;
    small = small || fabsf(a[j]) < kSmallA;
  }
  const bool accurate = !EULER && __any(small);
  const float bias2 = biasg ? biasg[d] * kLog2e : 0.f;
  const float dsk = Dg ? Dg[d] : 0.f;

  float4 hq[KB];
#pragma unroll
  for (int k = 0; k < KB; ++k) hq[k] = load_state4(S + ((bg * KB + k) * dim + d) * N + n0);
#pragma unroll
  for (int k = 0; k < KB; ++k) {
    const int64_t b = bg * KB + k;
    const int64_t row = b * dim + d;
    const float xv = to_f32(X[row]);
    float bv[4], cv[4];
    load4<Tin, true>(Bp + b * N + n0, n0, N, bv);
    load4<Tin, true>(Cp + b * N + n0, n0, N, cv);
    const float d2 = softplus_log2e(fmaf(to_f32(DT[row]), kLog2e, bias2));  // Delta * log2(e)
    const float dl = d2 * kLn2;
    float h[4] = {hq[k].x, hq[k].y, hq[k].z, hq[k].w};
    float yp = 0.f;
    auto update = [&](auto acc) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float arg = d2 * a[j];
        const float e = hw_exp2(arg);
        const float g = EULER ? dl : (decltype(acc)::value ? zoh_phi(e, arg, d2, rA[j]) : (e - 1.f) * rA[j]);
        h[j] = fmaf(e, h[j], g * bv[j] * xv);
        yp = fmaf(cv[j], h[j], yp);
      }
    };
    if (accurate)
      update(std::true_type{});
    else
      update(std::false_type{});
    store_state4(S + row * N + n0, h[0], h[1], h[2], h[3]);
    yp += __shfl_xor(yp, 1);
    yp += __shfl_xor(yp, 2);
    if (q == 0) {
      float yv = yp + dsk * xv;
      if (Z) yv *= silu(to_f32(Z[row]));
      store_val(&Y[row], yv);
    }
  }
}

namespace {

template <typename Tin, bool EU>
void launch_step16(const StepParams& p, hipStream_t s) {
  constexpr int KB = 4;
  const int64_t groups = p.batch / KB;
  const int64_t threads = groups * p.dim * 4;
  hipLaunchKernelGGL((step16_kernel<Tin, EU, KB>), dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0,
                     s, p.state, static_cast<const Tin*>(p.x), static_cast<const Tin*>(p.dt),
                     static_cast<const Tin*>(p.z), static_cast<const Tin*>(p.B), static_cast<const Tin*>(p.C), p.A,
                     p.Dskip, p.bias, static_cast<Tin*>(p.y), groups, p.dim);
}

template <typename Tin, int SPL, int LPR, bool VEC, int NF, bool EU>
void launch_step_one(const StepParams& p, hipStream_t s) {
  const int64_t rows = p.batch * p.dim;
  const int64_t threads = rows * LPR;
  if (p.conv_w) {
    hipLaunchKernelGGL((step_kernel<Tin, SPL, LPR, VEC, NF, EU, true>), dim3(static_cast<unsigned>((threads + 255) / 256)),
                       dim3(256), 0, s, p.state, static_cast<const Tin*>(p.x), static_cast<const Tin*>(p.dt),
                       static_cast<const Tin*>(p.z), static_cast<const Tin*>(p.B), static_cast<const Tin*>(p.C), p.A,
                       p.Dskip, p.bias, static_cast<Tin*>(p.y), rows, p.dim, p.N, p.conv_state, p.conv_w, p.conv_b,
                       p.dconv);
    return;
  }
  hipLaunchKernelGGL((step_kernel<Tin, SPL, LPR, VEC, NF, EU, false>), dim3(static_cast<unsigned>((threads + 255) / 256)),
                     dim3(256), 0, s, p.state, static_cast<const Tin*>(p.x), static_cast<const Tin*>(p.dt),
                     static_cast<const Tin*>(p.z), static_cast<const Tin*>(p.B), static_cast<const Tin*>(p.C), p.A,
                     p.Dskip, p.bias, static_cast<Tin*>(p.y), rows, p.dim, p.N, nullptr, nullptr, nullptr, 1);
}

template <typename Tin, bool EU>
void launch_step_t(const StepParams& p, bool vec, hipStream_t s) {
  if (p.N == 16 && vec && !p.conv_w && p.batch % 4 == 0) {
    launch_step16<Tin, EU>(p, s);
  } else if (p.N == 16 && vec) {
    // 4 states per lane: in-place float4 updates streamed at 5.4 TB/s against 5.0 with 8
    launch_step_one<Tin, 4, 4, true, 16, EU>(p, s);
  } else if (vec) {
    if (p.N <= 4) launch_step_one<Tin, 4, 1, true, 0, EU>(p, s);
    else if (p.N <= 8) launch_step_one<Tin, 8, 1, true, 0, EU>(p, s);
    else launch_step_one<Tin, 8, 2, true, 0, EU>(p, s);
  } else {
    if (p.N <= 4) launch_step_one<Tin, 4, 1, false, 0, EU>(p, s);
    else if (p.N <= 8) launch_step_one<Tin, 8, 1, false, 0, EU>(p, s);
    else launch_step_one<Tin, 8, 2, false, 0, EU>(p, s);
  }
}

}  // namespace

hipError_t launch_step(const StepParams& p, bool bf16, hipStream_t s) {
  const int64_t rows = p.batch * p.dim;
  if (rows <= 0) return hipSuccess;
  const uintptr_t bcal = bf16 ? 7 : 15;
  const bool vec = (p.N % 4 == 0) && ((reinterpret_cast<uintptr_t>(p.state) & 15) == 0) &&
                   ((reinterpret_cast<uintptr_t>(p.A) & 15) == 0) && ((reinterpret_cast<uintptr_t>(p.B) & bcal) == 0) &&
                   ((reinterpret_cast<uintptr_t>(p.C) & bcal) == 0);
  if (bf16)
    p.euler ? launch_step_t<bf16_t, true>(p, vec, s) : launch_step_t<bf16_t, false>(p, vec, s);
  else
    p.euler ? launch_step_t<float, true>(p, vec, s) : launch_step_t<float, false>(p, vec, s);
  return hipGetLastError();
}

}  // namespace sscan

// Forward selective scan on gfx950.
//
// What is computed (velog.io Mamba review, "Discretization" and section 3.2; page-3
// report sections 3 and 4.2): per batch row b and channel d, with Delta =
// softplus(dt + bias), Abar = exp(Delta A), Bbar = (exp(Delta A) - 1)/A * B,
// h_l = Abar h_{l-1} + Bbar x_l, y_l = (C_l . h_l + D x_l) * silu(z_l).
//
// Work decomposition.  A workgroup owns one (batch row, 64-channel tile, sequence
// segment).  Its NSPLIT waves split the N states, two states per wave, so the
// whole state of a channel stays in registers but spread over waves, and each
// lane of a wave is one channel.  The sequence is consumed in chunks of kChunk
// timesteps, software-pipelined with one barrier per chunk:
//   prologue   x, dt, z loaded coalesced along channels (each (l, d) once per
//              workgroup), Delta*log2(e) and x staged to LDS, silu(z) and D*x
//              kept in registers for the epilogue;
//   recurrence each wave reads (Delta, x) from LDS, B and C of its two states
//              arrive through scalar loads (uniform across the wave), updates its
//              states and writes a partial C.h to LDS;
//   epilogue   partials of all waves are summed, skip term and gate applied, y
//              stored coalesced.
// The state update uses h <- Abar (h + k) - k with k = x B / A, which equals
// Abar h + (Abar - 1) B x / A = Abar h + Bbar x: one add and one fma per state.
// A wave whose channels have some A == 0 switches to the explicit form with the
// Delta * B limit.
//
// Long sequences are split into segments (a two-level scan over the sequence):
// an aggregate pass scans each segment from a zero state and records its end
// state and sum of Delta; a carry pass combines them, segment by segment, into
// the state entering each segment (the product of Abar over a segment is
// exp(A * sum Delta)); the main pass then scans every segment from its carry.
#include "sscan_device.h"
#include "sscan_internal.h"

namespace sscan {

template <int P>
using Par = std::integral_constant<int, P>;

// Raw B and C words of a wave's two states at one timestep.
template <typename Tin, bool PAIR>
struct BCRaw;

// bf16, even N, 4-byte aligned B and C: the two states' values share one dword.
template <>
struct BCRaw<bf16_t, true> {
  uint32_t b, c;
  __device__ __forceinline__ void load(const bf16_t* __restrict__ B, const bf16_t* __restrict__ C, int64_t i0,
                                       int64_t i1) {
    (void)i1;
    b = reinterpret_cast<const uint32_t*>(B)[i0 >> 1];
    c = reinterpret_cast<const uint32_t*>(C)[i0 >> 1];
  }
  __device__ __forceinline__ float b0() const { return __uint_as_float(b << 16); }
  __device__ __forceinline__ float b1() const { return __uint_as_float(b & 0xffff0000u); }
  __device__ __forceinline__ float c0() const { return __uint_as_float(c << 16); }
  __device__ __forceinline__ float c1() const { return __uint_as_float(c & 0xffff0000u); }
};

template <typename Tin>
struct BCRaw<Tin, false> {
  Tin vb0, vb1, vc0, vc1;
  __device__ __forceinline__ void load(const Tin* __restrict__ B, const Tin* __restrict__ C, int64_t i0, int64_t i1) {
    vb0 = B[i0];
    vb1 = B[i1];
    vc0 = C[i0];
    vc1 = C[i1];
  }
  __device__ __forceinline__ float b0() const { return to_f32(vb0); }
  __device__ __forceinline__ float b1() const { return to_f32(vb1); }
  __device__ __forceinline__ float c0() const { return to_f32(vc0); }
  __device__ __forceinline__ float c1() const { return to_f32(vc1); }
};

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2).
// Remap the dispatch index so that consecutive logical blocks -- neighbouring
// channel tiles of one batch row, which read the same B and C rows -- run on
// the same XCD.  The map is a bijection of [0, nblk).
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t nblk) {
  constexpr int64_t kXcd = 8;
  const int64_t per = nblk / kXcd, rem = nblk % kXcd;
  const int64_t xcd = bid % kXcd, slot = bid / kXcd;
  return (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

template <typename Tin, int NSPLIT, bool AGG, bool PAIR>
__global__ __launch_bounds__(NSPLIT * 64) void fwd_kernel(FwdParams p) {
  constexpr int T = kChunk;
  constexpr int TPW = T / NSPLIT;  // prologue/epilogue timesteps per wave per chunk
  static_assert(T % NSPLIT == 0, "chunk must split evenly over waves");

  __shared__ float2 s_dx[2][T][kTile];
  __shared__ float s_yp[AGG ? 1 : 2][AGG ? 1 : NSPLIT][T][kTile];
  __shared__ float s_red[AGG ? NSPLIT : 1][kTile];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int64_t nseg_launched = AGG ? (p.nseg - 1) : p.nseg;
  int64_t blk = xcd_remap(blockIdx.x, p.ndtiles * p.batch * nseg_launched);
  const int64_t dtile = blk % p.ndtiles;
  blk /= p.ndtiles;
  const int64_t b = blk % p.batch;
  const int seg = static_cast<int>(blk / p.batch);

  const int64_t L = p.L, dim = p.dim;
  const int N = p.N;
  const int64_t l_begin = static_cast<int64_t>(seg) * p.seg_len;
  // Timestep counts within a segment fit in 32 bits (the host caps seqlen).
  const int seg_n = static_cast<int>(((l_begin + p.seg_len < L) ? l_begin + p.seg_len : L) - l_begin);
  const int nchunks = (seg_n + T - 1) / T;

  const int64_t d = dtile * kTile + lane;
  const bool dvalid = d < dim;
  const int64_t dd = dvalid ? d : dim - 1;

  // Scalar base pointers of this batch row; lanes add their channel.
  const int64_t tok0 = (b * L + l_begin) * dim + dtile * kTile;
  const Tin* __restrict__ Xb = static_cast<const Tin*>(p.x) + tok0;
  const Tin* __restrict__ DTb = static_cast<const Tin*>(p.dt) + tok0;
  const Tin* __restrict__ Zb = p.z ? static_cast<const Tin*>(p.z) + tok0 : nullptr;
  Tin* __restrict__ Yb = static_cast<Tin*>(p.y) + tok0;
  const Tin* __restrict__ Bb = static_cast<const Tin*>(p.B) + (b * L + l_begin) * N;
  const Tin* __restrict__ Cb = static_cast<const Tin*>(p.C) + (b * L + l_begin) * N;

  const float bias2 = p.bias ? p.bias[dd] * kLog2e : 0.f;
  const float dsk = p.Dskip ? p.Dskip[dd] : 0.f;
  const bool hasZ = (Zb != nullptr);

  // This wave's states n0, n0+1.  A state past N ("phantom", when 2*NSPLIT > N) gets
  // A = 1/A = 0, so Abar = 1, k = 0 and it stays exactly zero; B and C are read from
  // a clamped in-range index and never matter for it.
  const int n0 = 2 * w;
  const bool have0 = n0 < N, have1 = n0 + 1 < N;
  const int ni0 = have0 ? n0 : N - 1;
  const int ni1 = have1 ? n0 + 1 : N - 1;
  const float A0 = have0 ? p.A[dd * N + n0] : 0.f;
  const float A1 = have1 ? p.A[dd * N + n0 + 1] : 0.f;
  const float iA0 = (A0 != 0.f) ? 1.f / A0 : 0.f;
  const float iA1 = (A1 != 0.f) ? 1.f / A1 : 0.f;
  const float live0 = have0 ? 1.f : 0.f, live1 = have1 ? 1.f : 0.f;
  const bool zeroA = __any(dvalid && ((have0 && A0 == 0.f) || (have1 && A1 == 0.f)));

  float h0 = 0.f, h1 = 0.f;
  if constexpr (!AGG) {
    if (p.h_init && dvalid) {
      const float* hs = p.h_init + ((static_cast<int64_t>(seg) * p.batch + b) * dim + d) * N;
      if (have0) h0 = hs[n0];
      if (have1) h1 = hs[n0 + 1];
    }
  }

  Tin rx[TPW], rdt[TPW], rz[TPW];
  float eg[2][TPW], ed[2][TPW];
  float ssum = 0.f, scomp = 0.f;
  BCRaw<Tin, PAIR> bc[T];

  // Global loads of x, dt, z for this wave's prologue timesteps of chunk c.
  auto gload = [&](int c) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int l = c * T + w + NSPLIT * i;  // within the segment
      Tin a = Tin(0), e = Tin(0), f = Tin(0);
      if (l < seg_n) {
        const int64_t off = static_cast<int64_t>(l) * dim;
        if (dvalid) {
          a = Xb[off + lane];
          e = DTb[off + lane];
          if (!AGG && hasZ) f = Zb[off + lane];
        }
      }
      rx[i] = a;
      rdt[i] = e;
      rz[i] = f;
    }
  };

  // Raw B/C words of chunk c for this wave (index clamped into the segment).
  auto bcload = [&](int c) {
    const int lc = c * T;
    const int last = seg_n - 1 - lc;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int64_t row = static_cast<int64_t>(lc + (t < last ? t : last)) * N;
      bc[t].load(Bb, Cb, row + ni0, row + ni1);
    }
  };

  auto prologue = [&](auto pc, int c) {
    constexpr int P = decltype(pc)::value;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = w + NSPLIT * i;
      const bool lv = c * T + t < seg_n;
      const float xv = to_f32(rx[i]);  // zero when out of range
      float d2 = softplus_log2e(fmaf(to_f32(rdt[i]), kLog2e, bias2));
      d2 = lv ? d2 : 0.f;  // a padded step is the identity: Delta = 0, x = 0
      s_dx[P][t][lane] = make_float2(d2, xv);
      if constexpr (AGG) {
        const float yk = d2 - scomp;
        const float tk = ssum + yk;
        scomp = (tk - ssum) - yk;
        ssum = tk;
      } else {
        eg[P][i] = hasZ ? silu(to_f32(rz[i])) : 1.f;
        ed[P][i] = dsk * xv;
      }
    }
  };

  auto recur = [&](auto pc, int c) {
    constexpr int P = decltype(pc)::value;
    if (!zeroA) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const float2 v = s_dx[P][t][lane];
        const float q0 = bc[t].b0() * iA0;
        const float q1 = bc[t].b1() * iA1;
        const float e0 = hw_exp2(v.x * A0);
        const float e1 = hw_exp2(v.x * A1);
        const float k0 = v.y * q0;
        const float k1 = v.y * q1;
        h0 = fmaf(e0, h0 + k0, -k0);
        h1 = fmaf(e1, h1 + k1, -k1);
        if constexpr (!AGG) s_yp[P][w][t][lane] = fmaf(bc[t].c1(), h1, bc[t].c0() * h0);
      }
    } else {
      // Explicit form with the A == 0 limit: Bbar / B = (Abar - 1)/A, or Delta.
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const float2 v = s_dx[P][t][lane];
        const float dl = v.x * kLn2;
        const float e0 = hw_exp2(v.x * A0);
        const float g0 = live0 * ((A0 != 0.f) ? (e0 - 1.f) * iA0 : dl);
        h0 = fmaf(e0, h0, g0 * bc[t].b0() * v.y);
        const float e1 = hw_exp2(v.x * A1);
        const float g1 = live1 * ((A1 != 0.f) ? (e1 - 1.f) * iA1 : dl);
        h1 = fmaf(e1, h1, g1 * bc[t].b1() * v.y);
        if constexpr (!AGG) s_yp[P][w][t][lane] = fmaf(bc[t].c1(), h1, bc[t].c0() * h0);
      }
    }
    // Next chunk's B/C words: in flight across the barrier.  The scheduling
    // barrier keeps them from being hoisted over this chunk's uses, which would
    // hold two chunks of words in scalar registers at once.
    __builtin_amdgcn_sched_barrier(0);
    if (c + 1 < nchunks) bcload(c + 1);
  };

  auto epilogue = [&](auto pc, int c) {
    constexpr int P = decltype(pc)::value;
    if constexpr (!AGG) {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int t = w + NSPLIT * i;
        const int l = c * T + t;
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < NSPLIT; ++q) s += s_yp[P][q][t][lane];
        const float yv = (s + ed[P][i]) * eg[P][i];
        if (l < seg_n && dvalid) store_val(&Yb[static_cast<int64_t>(l) * dim + lane], yv);
      }
    }
  };

  if (nchunks > 0) {
    gload(0);
    bcload(0);
    prologue(Par<0>{}, 0);
    if (nchunks > 1) gload(1);
    __syncthreads();
    for (int c = 0; c < nchunks; c += 2) {
      if (c >= 1) epilogue(Par<1>{}, c - 1);
      if (c + 1 < nchunks) {
        prologue(Par<1>{}, c + 1);
        if (c + 2 < nchunks) gload(c + 2);
      }
      recur(Par<0>{}, c);
      __syncthreads();
      if (c + 1 < nchunks) {
        epilogue(Par<0>{}, c);
        if (c + 2 < nchunks) {
          prologue(Par<0>{}, c + 2);
          if (c + 3 < nchunks) gload(c + 3);
        }
        recur(Par<1>{}, c + 1);
        __syncthreads();
      }
    }
    if ((nchunks - 1) & 1)
      epilogue(Par<1>{}, nchunks - 1);
    else
      epilogue(Par<0>{}, nchunks - 1);
  }

  if constexpr (AGG) {
    if (dvalid) {
      float* ah = p.agg_h + ((static_cast<int64_t>(seg) * p.batch + b) * dim + d) * N;
      if (have0) ah[n0] = h0;
      if (have1) ah[n0 + 1] = h1;
    }
    s_red[w][lane] = ssum;
    __syncthreads();
    if (w == 0 && dvalid) {
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < NSPLIT; ++q) s += s_red[q][lane];
      p.agg_s[(static_cast<int64_t>(seg) * p.batch + b) * dim + d] = s;
    }
  } else {
    if (p.h_last && seg == p.nseg - 1 && dvalid) {
      float* hl = p.h_last + (b * dim + d) * N;
      if (have0) hl[n0] = h0;
      if (have1) hl[n0 + 1] = h1;
    }
  }
}

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
  for (int s = 0; s < nseg; ++s) {
    carry[static_cast<int64_t>(s) * total + i] = c;
    if (s + 1 < nseg)
      c = fmaf(hw_exp2(a * agg_s[static_cast<int64_t>(s) * batch * dim + bd]), c,
               agg_h[static_cast<int64_t>(s) * total + i]);
  }
}

__global__ __launch_bounds__(256) void fill_state_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                                         int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.f;
}

int fwd_nsplit(int N) {
  if (N <= 2) return 1;
  if (N <= 4) return 2;
  if (N <= 8) return 4;
  return 8;
}

namespace {

template <bool AGG>
hipError_t launch_fwd_impl(const FwdParams& p, bool bf16, hipStream_t s) {
  const int ns = fwd_nsplit(p.N);
  const int64_t nblocks = p.ndtiles * p.batch * (AGG ? (p.nseg - 1) : p.nseg);
  if (nblocks <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(nblocks)), block(ns * 64);
  const bool pair = bf16 && (p.N % 2 == 0) && ((reinterpret_cast<uintptr_t>(p.B) & 3) == 0) &&
                    ((reinterpret_cast<uintptr_t>(p.C) & 3) == 0);
#define SSCAN_LAUNCH(TIN, NS, PR) hipLaunchKernelGGL((fwd_kernel<TIN, NS, AGG, PR>), grid, block, 0, s, p)
#define SSCAN_BY_NS(TIN, PR)         \
  switch (ns) {                      \
    case 1: SSCAN_LAUNCH(TIN, 1, PR); break; \
    case 2: SSCAN_LAUNCH(TIN, 2, PR); break; \
    case 4: SSCAN_LAUNCH(TIN, 4, PR); break; \
    default: SSCAN_LAUNCH(TIN, 8, PR); break; \
  }
  if (!bf16) {
    SSCAN_BY_NS(float, false)
  } else if (pair) {
    SSCAN_BY_NS(bf16_t, true)
  } else {
    SSCAN_BY_NS(bf16_t, false)
  }
#undef SSCAN_BY_NS
#undef SSCAN_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_main(const FwdParams& p, bool bf16, hipStream_t s) { return launch_fwd_impl<false>(p, bf16, s); }

hipError_t launch_fwd_aggregate(const FwdParams& p, bool bf16, hipStream_t s) {
  return launch_fwd_impl<true>(p, bf16, s);
}

hipError_t launch_fwd_carry(const float* agg_h, const float* agg_s, const float* A, const float* h_init, float* carry,
                            int64_t batch, int64_t dim, int N, int nseg, hipStream_t s) {
  const int64_t total = batch * dim * N;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(carry_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s, agg_h, agg_s, A,
                     h_init, carry, batch, dim, N, nseg);
  return hipGetLastError();
}

hipError_t launch_fill_state(float* dst, const float* src, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_state_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, dst, src, n);
  return hipGetLastError();
}

}  // namespace sscan

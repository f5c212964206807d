// Forward selective scan on gfx950: the kernel template and its launch variants.
//
// What is computed (velog.io Mamba review, "Discretization" and section 3.2; page-3
// report sections 3 and 4.2): per batch row b and channel d, with Delta =
// softplus(dt + bias), Abar = exp(Delta A), Bbar = (exp(Delta A) - 1)/A * B,
// h_l = Abar h_{l-1} + Bbar x_l, y_l = (C_l . h_l + D x_l) * silu(z_l).
//
// Work decomposition.  A workgroup owns one (batch row, 64-channel tile, sequence
// segment).  Its NSPLIT waves split the N states, NPW (one or two) states per wave
// (NSPLIT is N / NPW rounded up to a power of two), so the whole state of a channel
// stays in registers but spread over waves, and each lane of a wave is one channel.
// The sequence is consumed in chunks of kChunk timesteps, software-pipelined with one
// barrier per chunk:
//   prologue   x, dt, z loaded coalesced along channels (each (l, d) once per
//              workgroup), Delta*log2(e) and x staged to LDS, silu(z) and D*x
//              kept in registers for the epilogue;
//   recurrence each wave reads (Delta, x) from LDS, the B value of its state
//              arrives through scalar loads (uniform across the wave), and the
//              state after every timestep is written to LDS;
//   epilogue   each wave reads back all N states of its own prologue timesteps,
//              forms C.h with the C row (scalar loads), adds the skip term,
//              applies the gate and stores y coalesced.  With two states per wave
//              the recurrence forms each wave's share of C.h instead (C through
//              scalar loads like B) and the epilogue adds NSPLIT partials; the
//              staging then fits two workgroups in a CU's LDS.
// The state update uses h <- Abar (h + k) - k with k = x B / A, which equals
// Abar h + (Abar - 1) B x / A = Abar h + Bbar x: one add and one fma per state.
// A wave whose channels have some |A| < kSmallA (A == 0 included) switches to the
// explicit form h <- Abar h + phi B x with the accurate phi of zoh_phi (Delta at A = 0).  With the Euler rule (Bbar = Delta B, the page-3 report's code,
// section 4.2) the prologue stages Delta*x instead of x and the update is
// h <- Abar h + (Delta x) B.
//
// Long sequences are split into segments (a two-level scan over the sequence):
// an aggregate pass scans each segment from a zero state and records its end
// state and sum of Delta; a carry pass combines them, segment by segment, into
// the state entering each segment (the product of Abar over a segment is
// exp(A * sum Delta)); the main pass then scans every segment from its carry.
#pragma once

#include "sscan_device.h"
#include "sscan_internal.h"

namespace sscan {

// B values of a wave's NPW states at one timestep, kept as raw scalar words.
// PAIR: even N and B and C aligned to two elements, so the wave's states sit in one
// aligned word (NPW = 2: both halves; NPW = 1: the half `sel` picks): a dword of two
// bf16, or a 64-bit pair of fp32.  Otherwise NPW elements are loaded one by one.
template <typename Tin, bool PAIR, int NPW>
struct BRaw {
  Tin v[NPW];
  __device__ __forceinline__ void load(const Tin* __restrict__ B, int64_t row, const int* joff) {
#pragma unroll
    for (int j = 0; j < NPW; ++j) v[j] = B[row + joff[j]];
  }
  __device__ __forceinline__ float get(int j, int) const { return to_f32(v[j]); }
  __device__ __forceinline__ void clear_missing(const bool* have) {
#pragma unroll
    for (int j = 0; j < NPW; ++j)
      if (!have[j]) v[j] = Tin(0);
  }
};

template <int NPW>
struct BRaw<bf16_t, true, NPW> {
  uint32_t wd;
  __device__ __forceinline__ void load(const bf16_t* __restrict__ B, int64_t row, const int*) {
    wd = *reinterpret_cast<const uint32_t*>(B + row);
  }
  // sel: 0 for the low half, 16 for the high half (used when NPW == 1).
  __device__ __forceinline__ float get(int j, int sel) const {
    if constexpr (NPW == 2) return __uint_as_float(j == 0 ? (wd << 16) : (wd & 0xffff0000u));
    return __uint_as_float((wd >> sel) << 16);
  }
  // N is even here, so a wave's two states are both real or both past N.
  __device__ __forceinline__ void clear_missing(const bool*) {}
};

// fp32 pairs: even N and 8-byte aligned B and C, so a wave's two states sit in one
// aligned 64-bit word, read by one scalar load instead of two.
template <int NPW>
struct BRaw<float, true, NPW> {
  float2 v;
  __device__ __forceinline__ void load(const float* __restrict__ B, int64_t row, const int*) {
    v = *reinterpret_cast<const float2*>(B + row);
  }
  __device__ __forceinline__ float get(int j, int sel) const {
    if constexpr (NPW == 2) return j == 0 ? v.x : v.y;
    return sel ? v.y : v.x;
  }
  __device__ __forceinline__ void clear_missing(const bool*) {}
};

// C row of one timestep (all N states) as float32, read through scalar loads.
template <typename Tin, bool PAIR, int NMAX>
__device__ __forceinline__ void load_c_row(const Tin* __restrict__ row, int N, float* c) {
  if constexpr (PAIR && std::is_same<Tin, float>::value) {
    const float2* r64 = reinterpret_cast<const float2*>(row);
#pragma unroll
    for (int k = 0; k < NMAX / 2; ++k) {
      const float2 wd = (2 * k < N) ? r64[k] : make_float2(0.f, 0.f);
      c[2 * k] = wd.x;
      c[2 * k + 1] = wd.y;
    }
  } else if constexpr (PAIR) {
    const uint32_t* r32 = reinterpret_cast<const uint32_t*>(row);
#pragma unroll
    for (int k = 0; k < NMAX / 2; ++k) {
      const uint32_t wd = (2 * k < N) ? r32[k] : 0u;
      c[2 * k] = __uint_as_float(wd << 16);
      c[2 * k + 1] = __uint_as_float(wd & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int n = 0; n < NMAX; ++n) c[n] = (n < N) ? to_f32(row[n]) : 0.f;
  }
}

// Register-only barriers for the optimizer (no memory effects, no instructions).
// opaque() hides how a scalar offset was computed, so per-timestep addresses are
// formed as constant offsets from one base instead of separate induction variables;
// after() also makes the offset depend on a vector value, so loads using it are
// issued only once that value (an LDS read) has arrived.  Only offsets are
// laundered, never pointers, so the compiler still sees which argument a load reads
// and can keep wave-uniform loads on the scalar unit.
__device__ __forceinline__ int64_t opaque(int64_t v) {
  asm("" : "+s"(v));
  return v;
}
__device__ __forceinline__ int64_t after(int64_t v, float dep) {
  asm("" : "+s"(v) : "v"(dep));
  return v;
}

// One workgroup: (batch row b, 64-channel tile, segment); NSPLIT waves x NPW states.
// MODE: kFwdOut (y and the final state), kFwdAgg (segment aggregates only: end state
// from a zero start and sum of Delta), kFwdCkpt (no y: the state entering every
// block of kBwdBlock steps is written to ckpt, for the backward pass), kFwdOutCkpt
// (both kFwdOut's and kFwdCkpt's outputs).  Launched are: the two-states-per-wave
// main pass of split grids (kFwdOut, kFwdOutCkpt), the aggregate pass, and the
// convolution prologue of split grids; the other launches run fwd_row_kernel
// (sscan_fwd_row.h).
// NFIX: N as a compile-time constant (0 = read it from the shape at run time).
// EULER: Bbar = Delta B instead of the zero-order hold.
// CONV: x is the raw input of a causal depthwise convolution over time (sh.dconv
// taps, conv_w [dim][dconv], optional conv_b [dim]) followed by SiLU, as in the
// page-3 report's MambaBlock (section 3, forward); the scan runs on its output.
// Inputs before the sequence start come from conv_s [batch][dim][dconv-1] (zeros
// when absent).
template <typename Tin, int NSPLIT, int NPW, int MODE, bool PAIR, int NFIX, bool EULER, bool CONV>
__global__ __launch_bounds__(NSPLIT * 64) void fwd_kernel(
    const Tin* __restrict__ xg, const Tin* __restrict__ dtg, const Tin* __restrict__ zg,
    const Tin* __restrict__ Bg, const Tin* __restrict__ Cg, const float* __restrict__ Ag,
    const float* __restrict__ Dg, const float* __restrict__ biasg, const float* __restrict__ h_init,
    Tin* __restrict__ yg, float* __restrict__ h_last, float* __restrict__ agg_h, float* __restrict__ agg_s,
    float* __restrict__ ckpt, const float* __restrict__ conv_w, const float* __restrict__ conv_b,
    const float* __restrict__ conv_s, FwdShape sh) {
  constexpr bool AGG = MODE == kFwdAgg;
  constexpr bool OUT = MODE == kFwdOut || MODE == kFwdOutCkpt;
  constexpr bool CKPT = MODE == kFwdCkpt || MODE == kFwdOutCkpt;
  constexpr int T = kChunk;
  constexpr int TPW = T / NSPLIT;  // prologue/epilogue timesteps per wave per chunk
  constexpr int H = T / 2;
  static_assert(T % NSPLIT == 0, "chunk must split evenly over waves");
  static_assert(NPW == 1 || NPW == 2, "one or two states per wave");

  // (Delta*log2(e), x) of each staged timestep (Delta*x instead of x for EULER),
  // interleaved so a lane reads both with one 64-bit access: on the training shape
  // that ran 2 % faster than two separate 32-bit arrays, whose extra read instructions
  // cost more than the wider accesses.
  __shared__ float2 s_dx[2][T][kTile];
  // States after each timestep, for the readout C.h done by the epilogue wave.
  // PART (output mode, two states per wave): each wave forms its own share of C.h in
  // the recurrence, so one partial per wave and timestep crosses LDS instead of one
  // state per state index; that halves this buffer and lets two workgroups share a CU.
  constexpr int NS = NSPLIT * NPW;
  constexpr bool PART = OUT && NPW == 2;
  __shared__ float s_h[OUT ? 2 : 1][OUT ? (PART ? NSPLIT : NS) : 1][T][kTile];
  // AGG: per-wave sums of Delta, in the state buffer (unused in that mode)
  static_assert(NSPLIT <= T, "s_red fits in s_h[0][0]");
  float (*s_red)[kTile] = s_h[0][0];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int64_t nseg_launched = AGG ? (sh.nseg - 1) : sh.nseg;
  int64_t blk = xcd_remap(blockIdx.x, sh.ndtiles * sh.batch * nseg_launched);
  const int64_t dtile = blk % sh.ndtiles;
  blk /= sh.ndtiles;
  const int64_t b = blk % sh.batch;
  const int seg = static_cast<int>(blk / sh.batch);

  const int64_t L = sh.L, dim = sh.dim;
  const int N = NFIX > 0 ? NFIX : sh.N;
  const int64_t l_begin = static_cast<int64_t>(seg) * sh.seg_len;
  // Timestep counts within a segment fit in 32 bits (the host caps seqlen).
  const int seg_n = static_cast<int>(((l_begin + sh.seg_len < L) ? l_begin + sh.seg_len : L) - l_begin);
  const int nchunks = (seg_n + T - 1) / T;
  const int nfull = seg_n / T;  // chunk nfull, if seg_n is not a multiple of T, is the tail

  const int64_t d = dtile * kTile + lane;
  const bool dvalid = d < dim;
  const int64_t dd = dvalid ? d : dim - 1;

  // Scalar base pointers of this (batch row, segment, channel tile); lanes add their channel.
  const int64_t tok0 = (b * L + l_begin) * dim + dtile * kTile;
  const Tin* __restrict__ Xb = xg + tok0;
  const Tin* __restrict__ DTb = dtg + tok0;
  const Tin* __restrict__ Zb = zg ? zg + tok0 : nullptr;
  Tin* __restrict__ Yb = yg + tok0;

  const float bias2 = biasg ? biasg[dd] * kLog2e : 0.f;
  const float dsk = Dg ? Dg[dd] : 0.f;
  const bool hasZ = (zg != nullptr);

  // This wave's states n0 .. n0+NPW-1.  A state past N ("phantom") gets A = 1/A = 0,
  // so Abar = 1, k = 0 and it stays exactly zero; its B and C come from an in-range
  // index and never matter.
  const int n0 = NPW * w;
  bool have[NPW];
  float Aj[NPW], iAj[NPW], live[NPW];
  int joff[NPW];
  // first element this wave reads in each B/C row
  const int nbase = PAIR ? ((n0 < N ? n0 : N - 2) & ~1) : (n0 < N ? n0 : N - 1);
  const int sel = PAIR ? ((n0 & 1) ? 16 : 0) : 0;
  bool anyzero = false;
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    have[j] = n0 + j < N;
    joff[j] = (have[j] ? n0 + j : N - 1) - nbase;
    Aj[j] = have[j] ? Ag[dd * N + n0 + j] : 0.f;
    iAj[j] = (Aj[j] != 0.f) ? 1.f / Aj[j] : 0.f;
    live[j] = have[j] ? 1.f : 0.f;
    anyzero = anyzero || (have[j] && fabsf(Aj[j]) < kSmallA);
  }
  // wave-uniform: some state of the wave's channels has |A| < kSmallA (A == 0 included)
  const bool smallA = __any(dvalid && anyzero);
  // B of this wave: element (l, nbase + o) of the segment sits at Bw[l * N + o].
  const Tin* __restrict__ Bw = Bg + (b * L + l_begin) * N + nbase;
  // C rows of the segment (the epilogue reads whole rows).
  const Tin* __restrict__ Cs = Cg + (b * L + l_begin) * N;
  // PART: C of this wave's states, addressed like B.
  const Tin* __restrict__ Cw = Cg + (b * L + l_begin) * N + nbase;

  float h[NPW];
#pragma unroll
  for (int j = 0; j < NPW; ++j) h[j] = 0.f;
  if constexpr (!AGG) {
    if (h_init && dvalid) {
      const float* hs = h_init + ((static_cast<int64_t>(seg) * sh.batch + b) * dim + d) * N;
#pragma unroll
      for (int j = 0; j < NPW; ++j)
        if (have[j]) h[j] = hs[n0 + j];
    }
  }

  Tin rx[TPW], rdt[TPW], rz[TPW];
  // CONV: raw inputs of the convolution window of each prologue timestep, and taps
  constexpr int KC = CONV ? kMaxConv : 1;
  Tin rxc[TPW][KC];
  float cw[KC];
  float cbias = 0.f;
  const int K = CONV ? sh.dconv : 1;
  const int lane_c = dvalid ? lane : 0;   // an in-range channel for lanes past dim
  if constexpr (CONV) {
#pragma unroll
    for (int k = 0; k < KC; ++k) cw[k] = (k < K) ? conv_w[dd * K + k] : 0.f;
    cbias = conv_b ? conv_b[dd] : 0.f;
  }
  float eg[2][TPW], ed[2][TPW];
  float ssum = 0.f, scomp = 0.f;
  BRaw<Tin, PAIR, NPW> bc[T];
  BRaw<Tin, PAIR, NPW> cc[PART ? T : 1];

  // Warm-up load of chunk c's B rows (and C rows in output mode) into the L2: the
  // waves read them later through scalar loads issued half a chunk ahead, whose misses
  // would otherwise wait on HBM.  One element per lane over the chunk's contiguous
  // rows (NSPLIT * 64 lanes cover both arrays: NSPLIT * NPW >= N); the value is only
  // kept alive, by the prologue that consumes the same chunk's x, dt and z.  Not in
  // the convolution variant, whose code the compiler then fails to build.
  Tin warm = Tin(0);
  auto bcwarm = [&](int c) {
    const int per = T * N;
    const int e = w * 64 + lane;
    const int rows = seg_n - c * T < T ? seg_n - c * T : T;
    const bool isc = OUT && e >= per;
    const int o = isc ? e - per : e;
    if ((isc || e < per) && o < rows * N) {
      const int64_t off = (b * L + l_begin + static_cast<int64_t>(c) * T) * N + o;
      warm = isc ? Cg[off] : Bg[off];
    }
  };
  auto keep_warm = [&]() {
    float v = to_f32(warm);
    asm volatile("" : "+v"(v));
  };

  // Global loads of x, dt, z for this wave's prologue timesteps of chunk c.
  auto gload = [&](int c) {
    if constexpr (!CONV) bcwarm(c);
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int l = c * T + w + NSPLIT * i;  // within the segment
      Tin a = Tin(0), e = Tin(0), f = Tin(0);
      if (l < seg_n) {
        const int64_t off = static_cast<int64_t>(l) * dim;
        if (dvalid) {
          if constexpr (!CONV) a = (Xb + off)[lane];
          e = (DTb + off)[lane];
          if (OUT && hasZ) f = (Zb + off)[lane];
        }
      }
      rx[i] = a;
      rdt[i] = e;
      rz[i] = f;
      if constexpr (CONV) {
        // window l - (K-1) .. l, loaded unconditionally from clamped in-range positions
        // (no per-lane branches); positions before the sequence start are replaced
        // from conv_s in the prologue, padded timesteps are discarded there
        const int64_t lg = l_begin + l;
        const int64_t lgc = lg < L ? lg : L - 1;
        const Tin* __restrict__ Xrow = xg + b * L * dim + dtile * kTile;
#pragma unroll
        for (int k = 0; k < KC; ++k) {
          const int back = (K - 1 - k) < 0 ? 0 : (K - 1 - k);
          const int64_t pos = lgc - (back <= lgc ? back : lgc);
          rxc[i][k] = (Xrow + pos * dim)[lane_c];
        }
      }
    }
  };

  // Raw B words of timesteps [H*hh, H*hh + H) of a full chunk c for this wave, into
  // bc[]: constant offsets from one scalar base.  `dep` orders the loads after an LDS
  // result (see the iteration).
  auto bcload_full = [&](int c, auto hc, float dep) {
    constexpr int HH = decltype(hc)::value;
    const int64_t off = after(opaque(static_cast<int64_t>(c) * T * N), dep);
    const Tin* Bc = Bw + off;
#pragma unroll
    for (int t = HH * H; t < (HH + 1) * H; ++t) bc[t].load(Bc, t * N, joff);
    if constexpr (PART) {
      const Tin* Cc = Cw + off;
#pragma unroll
      for (int t = HH * H; t < (HH + 1) * H; ++t) {
        cc[t].load(Cc, t * N, joff);
        cc[t].clear_missing(have);
      }
    }
  };
  // The same for the last, partial chunk: timesteps past the segment end read the
  // last row of the segment (they are identity steps whatever B holds).
  auto bcload_tail = [&](int c, float dep) {
    const int lc = c * T;
    const int last = seg_n - 1 - lc;
    const int64_t off = after(0, dep);
    const Tin* Bc = Bw + off;
#pragma unroll
    for (int t = 0; t < T; ++t) bc[t].load(Bc, static_cast<int64_t>(lc + (t < last ? t : last)) * N, joff);
    if constexpr (PART) {
      const Tin* Cc = Cw + off;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        cc[t].load(Cc, static_cast<int64_t>(lc + (t < last ? t : last)) * N, joff);
        cc[t].clear_missing(have);
      }
    }
  };

  auto prologue = [&](auto pc, int c) {
    constexpr int P = decltype(pc)::value;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = w + NSPLIT * i;
      const bool lv = c * T + t < seg_n;
      float xv = to_f32(rx[i]);  // zero when out of range
      if constexpr (CONV) {
        const int64_t l_glob = l_begin + c * T + t;
        float v[KC];
#pragma unroll
        for (int k = 0; k < KC; ++k) v[k] = to_f32(rxc[i][k]);
        if (l_glob < K - 1) {   // wave-uniform: the window reaches before the sequence
#pragma unroll
          for (int k = 0; k < KC; ++k) {
            const int64_t pos = l_glob - (K - 1) + k;
            if (pos < 0) v[k] = (conv_s && dvalid) ? conv_s[(b * dim + d) * (K - 1) + (K - 1) + pos] : 0.f;
          }
        }
        float acc = cbias;
#pragma unroll
        for (int k = 0; k < KC; ++k) acc = fmaf(cw[k], v[k], acc);   // taps past K are zero
        xv = lv ? silu(acc) : 0.f;   // a padded step stays the identity
      }
      float d2 = softplus_log2e(fmaf(to_f32(rdt[i]), kLog2e, bias2));
      d2 = lv ? d2 : 0.f;  // a padded step is the identity: Delta = 0, x = 0
      s_dx[P][t][lane] = make_float2(d2, EULER ? (d2 * kLn2) * xv : xv);
      if constexpr (AGG) {
        const float yk = d2 - scomp;
        const float tk = ssum + yk;
        scomp = (tk - ssum) - yk;
        ssum = tk;
      } else if constexpr (OUT) {
        eg[P][i] = hasZ ? silu(to_f32(rz[i])) : 1.f;
        ed[P][i] = dsk * xv;
      }
    }
    keep_warm();
  };

  // PART: this wave's share of C.h after timestep t, to LDS for the epilogue.
  auto stage = [&](auto pc, int t) {
    constexpr int P = decltype(pc)::value;
    if constexpr (PART) s_h[P][w][t][lane] = fmaf(cc[t].get(1, sel), h[1], cc[t].get(0, sel) * h[0]);
  };

  // One timestep of this wave's states, staged to LDS for the readout.  Fast form:
  // h <- Abar (h + k) - k with k = x B / A.  Accurate form (a wave with some
  // |A| < kSmallA): h <- Abar h + phi B x with phi = zoh_phi (Delta when A == 0).
  auto run_steps = [&](auto pc, auto hc, const float2* vx, const float (*ea)[NPW]) {
    constexpr int P = decltype(pc)::value;
    constexpr int HH = decltype(hc)::value;
    if constexpr (EULER) {
      // vx[t].y holds Delta * x; phantom states are never read back.
#pragma unroll
      for (int t = HH * H; t < (HH + 1) * H; ++t) {
#pragma unroll
        for (int j = 0; j < NPW; ++j) {
          h[j] = fmaf(ea[t][j], h[j], vx[t].y * bc[t].get(j, sel));
          if constexpr (OUT && !PART) s_h[P][n0 + j][t][lane] = h[j];
        }
        stage(pc, t);
      }
    } else if (!smallA) {
#pragma unroll
      for (int t = HH * H; t < (HH + 1) * H; ++t) {
#pragma unroll
        for (int j = 0; j < NPW; ++j) {
          const float q = bc[t].get(j, sel) * iAj[j];
          const float k = vx[t].y * q;
          h[j] = fmaf(ea[t][j], h[j] + k, -k);
          if constexpr (OUT && !PART) s_h[P][n0 + j][t][lane] = h[j];
        }
        stage(pc, t);
      }
    } else {
#pragma unroll
      for (int t = HH * H; t < (HH + 1) * H; ++t) {
#pragma unroll
        for (int j = 0; j < NPW; ++j) {
          const float g = live[j] * zoh_phi(ea[t][j], vx[t].x * Aj[j], vx[t].x, iAj[j]);
          h[j] = fmaf(ea[t][j], h[j], g * bc[t].get(j, sel) * vx[t].y);
          if constexpr (OUT && !PART) s_h[P][n0 + j][t][lane] = h[j];
        }
        stage(pc, t);
      }
    }
  };

  // Epilogue of chunk c for this wave's prologue timesteps: y = (C . h + D x) silu(z),
  // with the states h of all waves read back from LDS and the C row through scalar
  // loads.  g, dx: silu(z) and D*x of the same timesteps.
  auto epilogue = [&](auto pc, int c, const float* g, const float* dx) {
    constexpr int P = decltype(pc)::value;
    if constexpr (OUT) {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int t = w + NSPLIT * i;
        const int l = c * T + t;
        if (l < seg_n) {
          float sacc = dx[i];
          if constexpr (PART) {
            float pv[NSPLIT];
#pragma unroll
            for (int q = 0; q < NSPLIT; ++q) pv[q] = s_h[P][q][t][lane];
#pragma unroll
            for (int q = 0; q < NSPLIT; ++q)
              if (NPW * q < N) sacc += pv[q];
          } else {
            float hv[NS], cv[NS];
#pragma unroll
            for (int n = 0; n < NS; ++n) hv[n] = s_h[P][n][t][lane];
            load_c_row<Tin, PAIR, NS>(Cs + static_cast<int64_t>(l) * N, N, cv);
#pragma unroll
            for (int n = 0; n < NS; ++n)
              if (n < N) sacc = fmaf(cv[n], hv[n], sacc);
          }
          if (dvalid) store_val(&(Yb + static_cast<int64_t>(l) * dim)[lane], sacc * g[i]);
        }
      }
    }
  };
  auto read_dx = [&](auto pc, float2* vx) {
    constexpr int P = decltype(pc)::value;
#pragma unroll
    for (int t = 0; t < T - 1; ++t) vx[t] = s_dx[P][t][lane];
    __builtin_amdgcn_sched_barrier(0);
    vx[T - 1] = s_dx[P][T - 1][lane];  // issued last: once it has arrived, all have
    __builtin_amdgcn_sched_barrier(0);
  };

  // One iteration per chunk c, with one barrier at its end.  Scalar (B/C) and LDS
  // loads share one wait counter and scalar loads may complete out of order, so a
  // wait on an LDS result also waits for every scalar load in flight; the order
  // below keeps each scalar load ahead of the next LDS wait by a stretch of work:
  //   (Delta, x) of chunk c from LDS; prologue of chunk c+1 (consumes the global
  //   loads issued one iteration earlier); global loads of chunk c+2; the decays of
  //   chunk c; once the last LDS read has arrived, the scalar loads of the second
  //   half of this chunk's B/C; the first 8 timesteps; partials of chunk c-1 from
  //   LDS; the epilogue of chunk c-1 (stores y); the scalar loads of the first half
  //   of the next chunk's B/C (in flight across the barrier); the last 8 timesteps.
  auto iteration = [&](auto pc, auto tailc, int c) {
    constexpr int P = decltype(pc)::value;
    constexpr int Q = 1 - P;
    constexpr bool TAIL = decltype(tailc)::value;
    float2 vx[T];
    read_dx(pc, vx);
    float pg[TPW], pd[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      pg[i] = eg[Q][i];
      pd[i] = ed[Q][i];
    }
    if (c + 1 < nchunks) {
      prologue(Par<Q>{}, c + 1);
      if (c + 2 < nchunks) gload(c + 2);
    }
    float ea[T][NPW];  // Abar
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int j = 0; j < NPW; ++j) ea[t][j] = hw_exp2(vx[t].x * Aj[j]);
    if constexpr (TAIL)
      bcload_tail(c, vx[T - 1].y);
    else
      bcload_full(c, Par<1>{}, vx[T - 1].y);
    // state entering each half of the chunk: [batch][block][N][dim], block = index of
    // the kBwdBlock-step block in the sequence (two per chunk)
    static_assert(!CKPT || 2 * kBwdBlock == T, "checkpoints are taken at half chunks");
    auto checkpoint = [&](int half) {
      if constexpr (CKPT) {
        const int64_t blk = 2 * (l_begin / T + c) + half;
        if (dvalid && blk < sh.nblk) {
#pragma unroll
          for (int j = 0; j < NPW; ++j)
            if (have[j]) ckpt[((b * sh.nblk + blk) * N + n0 + j) * dim + d] = h[j];
        }
      }
    };
    checkpoint(0);
    run_steps(pc, Par<0>{}, vx, ea);
    __builtin_amdgcn_sched_barrier(0);
    if (OUT && c >= 1) epilogue(Par<Q>{}, c - 1, pg, pd);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!TAIL) {
      if (c + 1 < nfull) bcload_full(c + 1, Par<0>{}, h[0]);
    }
    __builtin_amdgcn_sched_barrier(0);
    checkpoint(1);
    run_steps(pc, Par<1>{}, vx, ea);
    __syncthreads();
  };

  if (nchunks > 0) {
    gload(0);
    prologue(Par<0>{}, 0);
    if (nchunks > 1) gload(1);
    if (nfull > 0) bcload_full(0, Par<0>{}, 0.f);
    __syncthreads();
    for (int c = 0; c < nfull; c += 2) {
      iteration(Par<0>{}, std::false_type{}, c);
      if (c + 1 < nfull) iteration(Par<1>{}, std::false_type{}, c + 1);
    }
    if (nfull < nchunks) {
      if (nfull & 1)
        iteration(Par<1>{}, std::true_type{}, nfull);
      else
        iteration(Par<0>{}, std::true_type{}, nfull);
    }
    if ((nchunks - 1) & 1)
      epilogue(Par<1>{}, nchunks - 1, eg[1], ed[1]);
    else
      epilogue(Par<0>{}, nchunks - 1, eg[0], ed[0]);
  }

  if constexpr (AGG) {
    if (dvalid) {
      float* ah = agg_h + ((static_cast<int64_t>(seg) * sh.batch + b) * dim + d) * N;
#pragma unroll
      for (int j = 0; j < NPW; ++j)
        if (have[j]) ah[n0 + j] = h[j];
    }
    s_red[w][lane] = ssum;
    __syncthreads();
    if (w == 0 && dvalid) {
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < NSPLIT; ++q) s += s_red[q][lane];
      agg_s[(static_cast<int64_t>(seg) * sh.batch + b) * dim + d] = s;
    }
  } else if constexpr (OUT) {
    if (h_last && seg == sh.nseg - 1 && dvalid) {
      float* hl = h_last + (b * dim + d) * N;
#pragma unroll
      for (int j = 0; j < NPW; ++j)
        if (have[j]) hl[n0 + j] = h[j];
    }
  }
}

template <typename Tin, int NS, int NPW, int MODE, bool PR, int NF, bool EU, bool CV>
void launch_one(const FwdParams& p, dim3 grid, hipStream_t s) {
  FwdShape sh{p.batch, p.L, p.dim, p.seg_len, p.ndtiles, p.nblk, p.rseg_len, p.N, p.nseg, p.dconv};
  hipLaunchKernelGGL((fwd_kernel<Tin, NS, NPW, MODE, PR, NF, EU, CV>), grid, dim3(NS * 64), 0, s,
                     static_cast<const Tin*>(p.x), static_cast<const Tin*>(p.dt), static_cast<const Tin*>(p.z),
                     static_cast<const Tin*>(p.B), static_cast<const Tin*>(p.C), p.A, p.Dskip, p.bias, p.h_init,
                     static_cast<Tin*>(p.y), p.h_last, p.agg_h, p.agg_s, p.ckpt, p.conv_w, p.conv_b, p.conv_s, sh);
}

template <typename Tin, int MODE, bool PR, bool EU, bool CV>
void launch_by_n(const FwdParams& p, dim3 grid, hipStream_t s) {
  if (p.npw == 2 && p.N >= 3) {
    switch (fwd_nsplit(2, p.N)) {
      case 2: launch_one<Tin, 2, 2, MODE, PR, 0, EU, CV>(p, grid, s); break;
      case 4: launch_one<Tin, 4, 2, MODE, PR, 0, EU, CV>(p, grid, s); break;
      default:
        if (p.N == 16)
          launch_one<Tin, 8, 2, MODE, PR, 16, EU, CV>(p, grid, s);
        else
          launch_one<Tin, 8, 2, MODE, PR, 0, EU, CV>(p, grid, s);
        break;
    }
    return;
  }
  // One state per wave: only the aggregate pass and the convolution prologue of split
  // grids with N < 3 still take it (other one-state launches run fwd_row_kernel;
  // launch_fwd_variant rejects them here).
  if constexpr (MODE == kFwdAgg || CV) {
    switch (fwd_nsplit(1, p.N)) {
      case 1: launch_one<Tin, 1, 1, MODE, PR, 0, EU, CV>(p, grid, s); break;
      case 2: launch_one<Tin, 2, 1, MODE, PR, 0, EU, CV>(p, grid, s); break;
      case 4: launch_one<Tin, 4, 1, MODE, PR, 0, EU, CV>(p, grid, s); break;
      case 8: launch_one<Tin, 8, 1, MODE, PR, 0, EU, CV>(p, grid, s); break;
      default:
        if (p.N == 16)
          launch_one<Tin, 16, 1, MODE, PR, 16, EU, CV>(p, grid, s);
        else
          launch_one<Tin, 16, 1, MODE, PR, 0, EU, CV>(p, grid, s);
        break;
    }
  }
}

// Launch of one (mode, discretization rule, convolution prologue) variant; each
// variant is instantiated in its own translation unit so the kernels compile in
// parallel.
template <int MODE, bool EU, bool CV>
hipError_t launch_fwd_variant(const FwdParams& p, bool bf16, hipStream_t s) {
  static_assert(MODE != kFwdCkpt, "the checkpoint pass runs fwd_row_kernel");
  if (!(MODE == kFwdAgg || CV) && !(p.npw == 2 && p.N >= 3)) return hipErrorInvalidValue;
  const int64_t nblocks = p.ndtiles * p.batch * (MODE == kFwdAgg ? (p.nseg - 1) : p.nseg);
  if (nblocks <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(nblocks));
  // two elements: 4 bytes for bf16, 8 for fp32
  const uintptr_t amask = bf16 ? 3 : 7;
  const bool pair = (p.N % 2 == 0) && ((reinterpret_cast<uintptr_t>(p.B) & amask) == 0) &&
                    ((reinterpret_cast<uintptr_t>(p.C) & amask) == 0);
  if (!bf16 && pair)
    launch_by_n<float, MODE, true, EU, CV>(p, grid, s);
  else if (!bf16)
    launch_by_n<float, MODE, false, EU, CV>(p, grid, s);
  else if (pair)
    launch_by_n<bf16_t, MODE, true, EU, CV>(p, grid, s);
  else
    launch_by_n<bf16_t, MODE, false, EU, CV>(p, grid, s);
  return hipGetLastError();
}

}  // namespace sscan

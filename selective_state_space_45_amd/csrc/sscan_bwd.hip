// Backward pass of the selective scan on gfx950: gradients of a scalar loss with
// respect to x, dt, z, A, B, C, D, the step-size bias and the initial state.
//
// The forward definition (velog.io Mamba review, "Discretization" and section 3.2;
// page-3 report sections 3 and 4.2) differentiated by the chain rule and run
// backwards in time: the reverse recurrence the page-3 report's pscan_rev serves
// (section 4.1), with the forward intermediates recomputed rather than stored (the
// recomputation that the lengnian.github.io notes, "Part3: Mamba - A Selective SSM",
// list in the hardware-aware algorithm).
// Per batch row and channel, with g_l the gradient reaching the state h_l:
//   g_l     = gyo_l C_l + Abar_{l+1} g_{l+1},   gyo_l = dy_l silu(z_l)
//   dx_l    = gyo_l D + sum_n g_l phi_l B_l,    dB_l = sum_d g_l phi_l x_l,
//   dC_l    = sum_d gyo_l h_l,                  dz_l = dy_l yo_l silu'(z_l)
//   dDelta  = sum_n g_l (A Abar h_{l-1} + dphi/dDelta B_l x_l),  ddt = dDelta sigmoid(dt + bias)
//   dA      = sum_{b,l} g_l (Delta Abar h_{l-1} + dphi/dA B_l x_l)
// with phi = Bbar / B: (Abar - 1)/A for the zero-order hold (dphi/dDelta = Abar,
// dphi/dA = (Delta Abar - phi)/A, evaluated by its Taylor series in u = Delta A when
// |u| < 0.5), Delta for the Euler rule (dphi/dDelta = 1, dphi/dA = 0).  Waves with some
// |A| < kSmallA form phi itself with zoh_phi (accurate as u -> 0); the others use
// forms that divide by A, exact in exact arithmetic and accurate for |A| >= kSmallA.
//
// Work decomposition: a workgroup owns (batch row, 64-channel tile, reverse
// segment); lane = channel, and each wave owns kBwdSpw (two) states (a wave's sums
// over its states are formed in registers, so only one partial per wave crosses
// LDS).  A checkpoint pass of the forward kernel has stored the state entering
// every kBwdBlock-step (8-step) block.  The workgroup walks its blocks from last to
// first, with each block's global inputs loaded one block ahead; per block:
//   P1  each wave loads its timesteps' x, dt, z, dy; Delta, x and gyo are staged to
//       LDS, with the block's B and C rows;
//   P2  each wave recomputes its state over the block from the checkpoint (the
//       states kept in registers); C.h goes to LDS for the readout yo, and the
//       per-channel terms of dC are summed across lanes;
//   P3  (gate only) each wave forms yo and dz for its timesteps;
//   P4  each wave runs the reverse recurrence over the block (decays recomputed),
//       writing its terms of dx and dDelta to LDS, accumulating dA, and summing the
//       terms of dB across lanes;
//   P5  each wave sums the terms over states for its timesteps and stores dx, ddt.
// dB and dC leave as per-tile partial sums, dA, dD and dbias as per-batch-row
// partial sums; small reduction kernels finish them in a fixed order.
#include <type_traits>

#include "selscan.h"
#include "sscan_device.h"
#include "sscan_internal.h"
#include "sscan_lanes.h"

namespace sscan {

namespace {

// Value of v in the lane that DPP control CTRL selects (a permutation within rows).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppRowRor8 = 0x128;        // lane i <- row lane (i + 8) mod 16: partner i ^ 8
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- 7 - i within each 8 lanes: partner i ^ 7
constexpr int kDppQuadXor2 = 0x4e;        // quad_perm [2,3,0,1]
constexpr int kDppQuadXor1 = 0xb1;        // quad_perm [1,0,3,2]

__device__ __forceinline__ void unpack(const float4& v, float* o) {
  o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
__device__ __forceinline__ void unpack(const float2& v, float* o) {
  o[0] = v.x; o[1] = v.y;
}

// One halving step of a butterfly reduce-scatter through a DPP permutation that
// pairs every lane with a partner whose BIT differs: lanes with BIT clear keep
// elements [0, half), the others [half, 2 half), each summed over the pair.
template <int CTRL, int BIT, int HALF>
__device__ __forceinline__ void halve_dpp(float* v, int lane) {
  const bool upper = (lane & BIT) != 0;
#pragma unroll
  for (int k = 0; k < HALF; ++k) {
    const float keep = upper ? v[k + HALF] : v[k];
    const float send = upper ? v[k] : v[k + HALF];
    v[k] = keep + dpp<CTRL>(send);
  }
}

// Sum of v[0..31] over the 64 lanes of a wave, as a reduce-scatter: afterwards
// lane L holds in v[0] the total of element L >> 1 (both lanes of a pair agree).
// The two wide steps use the gfx950 half-swaps (lane i <-> i ^ 32, i ^ 16), the
// narrow ones DPP row permutations: no LDS and no address registers.
__device__ __forceinline__ void lane_reduce32(float* v, int lane) {
#pragma unroll
  for (int k = 0; k < 16; ++k) {   // partner i ^ 32: lanes 0..31 keep k, 32..63 keep k + 16
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[k]), __float_as_uint(v[k + 16]), false, false);
    v[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {    // partner i ^ 16: rows 0 and 2 keep k, rows 1 and 3 keep k + 8
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[k]), __float_as_uint(v[k + 8]), false, false);
    v[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  halve_dpp<kDppRowRor8, 8, 4>(v, lane);
  halve_dpp<kDppRowHalfMirror, 4, 2>(v, lane);
  halve_dpp<kDppQuadXor2, 2, 1>(v, lane);
  v[0] += dpp<kDppQuadXor1>(v[0]);
}

// The halvings through row_ror:8 (partner lane ^ 8) and row_half_mirror (partner
// ^ 7 within each half row) pair lanes in different groups of four, so each output
// register is written by two adds masked to lane groups (bank_mask), one per half,
// with no per-lane selects: 2 VALU per output instead of 3.  Lanes with the bit clear
// keep the lower half of the elements, as halve_dpp does.  Inline assembly (the
// compiler has no masked-add builtin); each block starts with the two wait states a
// DPP read of a VGPR written by the preceding VALU instruction requires.  All 64
// lanes must be active.
__device__ __forceinline__ void halve_ror8_2(float* v) {
  float o0, o1;
  asm("s_nop 1\n\t"
      "v_add_f32_dpp %0, %2, %2 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %0, %4, %4 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %1, %3, %3 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %1, %5, %5 row_ror:8 row_mask:0xf bank_mask:0xc"
      : "=&v"(o0), "=&v"(o1)
      : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]));
  v[0] = o0;
  v[1] = o1;
}
__device__ __forceinline__ void halve_mirror_1(float* v) {
  float o0;
  asm("s_nop 1\n\t"
      "v_add_f32_dpp %0, %1, %1 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %0, %2, %2 row_half_mirror row_mask:0xf bank_mask:0xa"
      : "=&v"(o0)
      : "v"(v[0]), "v"(v[1]));
  v[0] = o0;
}

// Sum of v[0..15] over the 64 lanes of a wave, as a reduce-scatter: afterwards lane
// L holds in v[0] the total of element L >> 2 (all four lanes of a quad agree).
__device__ __forceinline__ void lane_reduce16(float* v, int lane) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[k]), __float_as_uint(v[k + 8]), false, false);
    v[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[k]), __float_as_uint(v[k + 4]), false, false);
    v[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  (void)lane;
  halve_ror8_2(v);
  halve_mirror_1(v);
  v[0] += dpp<kDppQuadXor2>(v[0]);
  v[0] += dpp<kDppQuadXor1>(v[0]);
}

// Reduce-scatter of S * kBwdBlock values: element k ends in lanes (k << SH) .. ((k+1) << SH) - 1.
template <int NV>
__device__ __forceinline__ void lane_reduce(float* v, int lane) {
  if constexpr (NV == 32)
    lane_reduce32(v, lane);
  else
    lane_reduce16(v, lane);
}

// (u e^u - e^u + 1) / u^2 by its Taylor series sum_k (k+1) u^k / (k+2)!, |u| < 0.5.
__device__ __forceinline__ float dphi1_series(float u) {
  float r = 1.f / 5760.f;
  r = fmaf(u, r, 1.f / 840.f);
  r = fmaf(u, r, 1.f / 144.f);
  r = fmaf(u, r, 1.f / 30.f);
  r = fmaf(u, r, 1.f / 8.f);
  r = fmaf(u, r, 1.f / 3.f);
  return fmaf(u, r, 0.5f);
}

}  // namespace

// States per wave of the backward kernel, and waves per workgroup for a given N.
constexpr int kBwdSpw = 2;
inline int bwd_waves(int N) {
  int w = 1;
  while (w * kBwdSpw < N) w <<= 1;
  return w;
}

template <typename Tin, int NW, int NFIX, bool EULER>
__global__ __launch_bounds__(NW * 64) void bwd_kernel(
    const Tin* __restrict__ xg, const Tin* __restrict__ dtg, const Tin* __restrict__ zg,
    const Tin* __restrict__ Bg, const Tin* __restrict__ Cg, const Tin* __restrict__ dyg,
    const float* __restrict__ Ag, const float* __restrict__ Dg, const float* __restrict__ biasg,
    const float* __restrict__ dlast, const float* __restrict__ gin, const float* __restrict__ ckpt,
    Tin* __restrict__ dxg, Tin* __restrict__ ddtg, Tin* __restrict__ dzg, float* __restrict__ gBp,
    float* __restrict__ gCp, float* __restrict__ gAp, float* __restrict__ gDp, float* __restrict__ gbp,
    float* __restrict__ dh0, BwdShape sh) {
  constexpr int T = kBwdBlock;        // timesteps per block (one checkpoint each)
  constexpr int S = kBwdSpw;          // states per wave
  constexpr int NSP = NW * S;         // states covered (N rounded up)
  constexpr int TPW = T / NW;         // prologue / epilogue timesteps per wave
  static_assert(T * S == 32 || T * S == 16, "a block's terms of one wave fill one lane reduction");
  constexpr int NV = T * S;                 // values per lane reduction
  constexpr int SH = NV == 32 ? 1 : 2;      // lanes per reduced element: 1 << SH
  static_assert(T % NW == 0, "block must split evenly over waves");

  // staging of one block, double-buffered (P1 of block j-1 overlaps P5 of block j)
  __shared__ float s_d2[2][T][kTile];     // Delta * log2(e)
  __shared__ float s_xv[2][T][kTile];     // x
  __shared__ float s_go[2][T][kTile];     // gyo = dy * silu(z)
  // B and C of the block, S consecutive states per vector
  using VS = typename std::conditional<S == 4, float4, float2>::type;
  __shared__ VS s_B[2][T][NSP / S];
  __shared__ VS s_C[2][T][NSP / S];
  // per-wave partial sums over its states: C.h (readout), dx terms, dDelta terms
  __shared__ float s_r0[NW][T][kTile];
  __shared__ float s_r1[NW][T][kTile];
  __shared__ float s_r2[NW][T][kTile];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tid = threadIdx.x;

  int64_t blk = xcd_remap(blockIdx.x, sh.ndtiles * sh.batch * sh.nseg);
  const int64_t dtile = blk % sh.ndtiles;
  blk /= sh.ndtiles;
  const int64_t b = blk % sh.batch;
  const int seg = static_cast<int>(blk / sh.batch);
  const int64_t L = sh.L, dim = sh.dim;
  const int N = NFIX > 0 ? NFIX : sh.N;
  const int dim32 = static_cast<int>(dim);   // T * dim < 2^31 (checked by the host)

  const int64_t d = dtile * kTile + lane;
  const bool dvalid = d < dim;
  const int64_t dd = dvalid ? d : dim - 1;
  const bool hasZ = zg != nullptr;
  const float bias2 = biasg ? biasg[dd] * kLog2e : 0.f;
  const float dsk = Dg ? Dg[dd] : 0.f;

  // this wave's states n0 .. n0 + S - 1; phantom states (n >= N) get A = 0 and stay
  // out of every output
  const int n0 = S * w;
  // gradient entering the end of this segment ([batch][dim][N] slice): the carry of
  // the sequence split, or dLoss/d(last state) for the last segment
  const float* g_in = nullptr;
  if (gin)
    g_in = gin + static_cast<int64_t>(seg) * sh.batch * dim * N;
  else if (seg == sh.nseg - 1)
    g_in = dlast;
  float An[S], iAn[S], G[S], gA[S];
  bool anyzero = false;
#pragma unroll
  for (int q = 0; q < S; ++q) {
    const bool have = n0 + q < N;
    An[q] = have ? Ag[dd * N + n0 + q] : 0.f;
    iAn[q] = (An[q] != 0.f) ? 1.f / An[q] : 0.f;
    anyzero = anyzero || (have && fabsf(An[q]) < kSmallA);
    G[q] = (g_in && have && dvalid) ? g_in[(b * dim + d) * N + n0 + q] : 0.f;
    gA[q] = 0.f;
  }
  // wave-uniform: some state of the wave's channels has |A| < kSmallA (A == 0
  // included), where the k-form's rounding error would matter; those waves take the
  // explicit forms with the accurate zoh_phi
  const bool smallA = __any(dvalid && anyzero);

  const int64_t tok_b = b * L * dim + dtile * kTile;  // token offset of (b, l = 0, this tile)
  float e_sig[TPW], e_gz[TPW];                       // epilogue values of this wave's timesteps
  float accD = 0.f, accBias = 0.f;

  // Global inputs of one block, loaded one block ahead of their use: x, dt, z, dy of
  // this wave's timesteps, one B and one C element of the block's rows, and this
  // wave's checkpoint states.
  Tin r_x[TPW], r_dt[TPW], r_z[TPW], r_dy[TPW];
  Tin r_b = Tin(0), r_c = Tin(0);
  float r_ck[S];
  const int bc_t = tid / NSP, bc_n = tid - (tid / NSP) * NSP;   // B/C element this thread stages
  const bool bc_stager = tid < T * NSP;
  auto gload = [&](int64_t j) {
    const int64_t l0 = j * T;
    const int cnt = static_cast<int>((L - l0) < T ? (L - l0) : T);
    const int64_t base = tok_b + l0 * dim;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = w + NW * i;
      Tin a = Tin(0), e = Tin(0), f = Tin(0), g = Tin(0);
      if (dvalid && t < cnt) {
        const int off = t * dim32 + lane;
        a = (xg + base)[off];
        e = (dtg + base)[off];
        g = (dyg + base)[off];
        if (hasZ) f = (zg + base)[off];
      }
      r_x[i] = a;
      r_dt[i] = e;
      r_z[i] = f;
      r_dy[i] = g;
    }
    r_b = Tin(0);
    r_c = Tin(0);
    if (bc_stager && bc_n < N && bc_t < cnt) {
      const int64_t r = (b * L + l0 + bc_t) * N + bc_n;
      r_b = Bg[r];
      r_c = Cg[r];
    }
    const float* ck = ckpt + ((b * sh.nblk + j) * N) * dim + dtile * kTile;
#pragma unroll
    for (int q = 0; q < S; ++q) r_ck[q] = (n0 + q < N && dvalid) ? ck[(n0 + q) * dim + lane] : 0.f;
  };

  // P1: from the prefetched inputs of block j: Delta, x, gyo to LDS buffer j & 1 with
  // the block's B and C rows; silu'(z) and sigmoid(dt + bias) kept for P5.
  float h_next[S];
  auto prologue = [&](int64_t j) {
    const int pb = static_cast<int>(j & 1);
    const int64_t l0 = j * T;
    const int cnt = static_cast<int>((L - l0) < T ? (L - l0) : T);
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = w + NW * i;
      const float xv = to_f32(r_x[i]), zv = to_f32(r_z[i]), gy = to_f32(r_dy[i]);
      const float v2 = fmaf(to_f32(r_dt[i]), kLog2e, bias2);
      float gyo = gy, gz = 0.f;
      if (hasZ) {
        const float sg = hw_rcp(1.f + hw_exp2(-zv * kLog2e));
        gyo = gy * (zv * sg);
        gz = gy * sg * fmaf(zv, 1.f - sg, 1.f);   // dy * silu'(z)
      }
      s_d2[pb][t][lane] = (t < cnt) ? softplus_log2e(v2) : 0.f;
      s_xv[pb][t][lane] = xv;
      s_go[pb][t][lane] = gyo;
      e_gz[i] = gz;
      e_sig[i] = hw_rcp(1.f + hw_exp2(-v2));  // sigmoid(dt + bias) = softplus'
    }
    if (bc_stager) {
      reinterpret_cast<float*>(s_B[pb])[tid] = to_f32(r_b);
      reinterpret_cast<float*>(s_C[pb])[tid] = to_f32(r_c);
    }
#pragma unroll
    for (int q = 0; q < S; ++q) h_next[q] = r_ck[q];
  };

  const int64_t nblk = sh.nblk;
  const int64_t jbeg = static_cast<int64_t>(seg) * sh.seg_blocks;
  const int64_t jend = (jbeg + sh.seg_blocks < nblk) ? jbeg + sh.seg_blocks : nblk;
  if (jend > jbeg) {
    gload(jend - 1);
    prologue(jend - 1);
    if (jend - 2 >= jbeg) gload(jend - 2);
  }
  for (int64_t j = jend - 1; j >= jbeg; --j) {
    const int pb = static_cast<int>(j & 1);
    const int64_t l0 = j * T;
    const int cnt = static_cast<int>((L - l0) < T ? (L - l0) : T);
    const int64_t tok_blk = tok_b + l0 * dim;
    const int64_t part = (dtile * sh.batch + b) * N * L + l0;   // + n * L + t: partials of dB, dC
    float h[S];
#pragma unroll
    for (int q = 0; q < S; ++q) h[q] = h_next[q];
    __syncthreads();
    // this wave's B and C pairs of the block, addressed from a vector register (a zero
    // the compiler cannot see through), so that the per-step reads use immediate
    // offsets instead of re-copying a scalar address into a vector register each step
    int vzero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(vzero));
    const VS* __restrict__ sBw = reinterpret_cast<const VS*>(reinterpret_cast<const char*>(&s_B[pb][0][w]) + vzero);
    const VS* __restrict__ sCw = reinterpret_cast<const VS*>(reinterpret_cast<const char*>(&s_C[pb][0][w]) + vzero);

    // ---- P2: recompute the block's states from the checkpoint; partial C.h of the
    // readout to LDS; terms of dC summed across lanes ----
    float hist[S][T];   // state entering each step
    float ahist[S][T];  // Abar of each step, reused by the reverse recurrence
    {
      float red[S * T];
      auto recompute = [&](auto safe) {
        constexpr bool SAFE = decltype(safe)::value;
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const float d2 = s_d2[pb][t][lane];
          const float xv = s_xv[pb][t][lane];
          const float go = s_go[pb][t][lane];
          float bq[S], cq[S];
          unpack(sBw[t * (NSP / S)], bq);
          unpack(sCw[t * (NSP / S)], cq);
          float yo = 0.f;
#pragma unroll
          for (int q = 0; q < S; ++q) {
            const float a = hw_exp2(d2 * An[q]);
            ahist[q][t] = a;
            hist[q][t] = h[q];
            if constexpr (EULER) {
              h[q] = fmaf(a, h[q], (d2 * kLn2) * xv * bq[q]);
            } else if constexpr (!SAFE) {
              const float k = xv * bq[q] * iAn[q];
              h[q] = fmaf(a, h[q] + k, -k);
            } else {
              const float g = zoh_phi(a, d2 * An[q], d2, iAn[q]);
              h[q] = fmaf(a, h[q], g * bq[q] * xv);
            }
            red[q * T + t] = go * h[q];
            yo = fmaf(cq[q], h[q], yo);
          }
          s_r0[w][t][lane] = yo;
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      if (EULER || !smallA)
        recompute(std::false_type{});
      else
        recompute(std::true_type{});
      lane_reduce<NV>(red, lane);
      if ((lane & ((1 << SH) - 1)) == 0) {
        const int k = lane >> SH, q = k / T, t = k % T;
        if (n0 + q < N && t < cnt) gCp[part + (n0 + q) * L + t] = red[0];
      }
    }

    // ---- P4: reverse recurrence over the block (decays recomputed); partial sums
    // of the dx and dDelta terms to LDS, dA accumulated, terms of dB summed across
    // lanes ----
    {
      float red[S * T];
#pragma unroll
      for (int t = T - 1; t >= 0; --t) {
        const float go = s_go[pb][t][lane];
        const float d2 = s_d2[pb][t][lane];
        const float xv = s_xv[pb][t][lane];
        float bq[S], cq[S];
        unpack(sBw[t * (NSP / S)], bq);
        unpack(sCw[t * (NSP / S)], cq);
        const float delta = d2 * kLn2;
        float r1 = 0.f, r2 = 0.f;
        // both states of the step in one block, behind one wave-uniform branch per step
        // (a branch per state kept the two states' chains from interleaving and cost a
        // taken branch and a jump per state-step on the fast path)
        auto states = [&](auto slowc) __attribute__((always_inline)) {
          constexpr bool SLOW = decltype(slowc)::value;
#pragma unroll
          for (int q = 0; q < S; ++q) {
            const float a = ahist[q][t];
            const float hp = hist[q][t];
            const float gh = fmaf(go, cq[q], G[q]);
            const float bx = bq[q] * xv;
            // hn = h_l, the state after the step: h_l = Abar h_{l-1} + phi B x
            const float hn = (t + 1 < T) ? hist[q][t + 1] : h[q];
            float gphi;
            const float Gn = a * gh;
            if constexpr (EULER) {
              gphi = gh * delta;
              r2 = fmaf(gh, fmaf(An[q] * a, hp, bx), r2);
              gA[q] = fmaf(gh, delta * a * hp, gA[q]);
            } else {
              if constexpr (!SLOW) {
                // d h_l / d Delta = Abar (A h_{l-1} + B x) = A hn + B x = A (hn + k) and
                // d h_l / d A = Delta Abar (h_{l-1} + k) - phi k = Delta (hn + k) - phi k,
                // with k = B x / A: both terms share q = gh (hn + k).  gh phi = (Abar gh
                // - gh) / A, so phi is never formed.  The term (Delta Abar - phi) k
                // cancels for small Delta A, but only down to a few ulp of Delta k, the
                // size of the leading term (this form serves |A| >= kSmallA only)
                gphi = (Gn - gh) * iAn[q];
                const float k = bx * iAn[q];
                const float qh = gh * (hn + k);
                r2 = fmaf(An[q], qh, r2);
                gA[q] = fmaf(delta, qh, gA[q]);
                gA[q] = fmaf(-gphi, k, gA[q]);
              } else {
                // d h_l / d Delta = A hn + B x, formed directly (k = B x / A is large here)
                r2 = fmaf(gh, fmaf(An[q], hn, bx), r2);
                const float phi = zoh_phi(a, d2 * An[q], d2, iAn[q]);
                gphi = gh * phi;
                // a wave with some small |A|: dphi/dA = Delta^2 (u e^u - e^u + 1)/u^2,
                // u = Delta A, from its series for |u| < 0.5 and its closed form
                // otherwise; both are computed (each finite everywhere) and blended, so
                // no per-lane branch splits the step
                const float u = delta * An[q];
                const float ser = delta * delta * dphi1_series(fmaxf(fminf(u, 0.5f), -0.5f));
                const float dir = (delta * a - phi) * iAn[q];
                const float wsel = (fabsf(u) < 0.5f) ? 1.f : 0.f;
                const float dphi_dA = fmaf(wsel, ser - dir, dir);
                gA[q] = fmaf(gh, fmaf(delta * a, hp, dphi_dA * bx), gA[q]);
              }
            }
            red[q * T + t] = gphi * xv;
            r1 = fmaf(gphi, bq[q], r1);
            G[q] = Gn;
          }
        };
        if (EULER || !smallA)
          states(std::false_type{});
        else
          states(std::true_type{});
        s_r1[w][t][lane] = r1;
        s_r2[w][t][lane] = r2;
        // dA is needed only after the last block; without this anchor the compiler
        // sinks its update out of the step and keeps every step's terms alive
#pragma unroll
        for (int q = 0; q < S; ++q) asm volatile("" : "+v"(gA[q]));
        __builtin_amdgcn_sched_barrier(0);
      }
      lane_reduce<NV>(red, lane);
      if ((lane & ((1 << SH) - 1)) == 0) {
        const int k = lane >> SH, q = k / T, t = k % T;
        if (n0 + q < N && t < cnt) gBp[part + (n0 + q) * L + t] = red[0];
      }
    }
    if (j == 0 && dh0 && dvalid) {
#pragma unroll
      for (int q = 0; q < S; ++q)
        if (n0 + q < N) dh0[(b * dim + d) * N + n0 + q] = G[q];
    }
    __syncthreads();

    // ---- P5: sums over states; store dz, dx, ddt.  Then P1 of the next block into
    // the other staging buffer ----
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = w + NW * i;
      if (dvalid && t < cnt) {
        const float go = s_go[pb][t][lane];
        const float xv = s_xv[pb][t][lane];
        float gx = go * dsk, gd = 0.f, yo = dsk * xv;
#pragma unroll
        for (int q = 0; q < NW; ++q) {
          yo += s_r0[q][t][lane];
          gx += s_r1[q][t][lane];
          gd += s_r2[q][t][lane];
        }
        const float gdt = gd * e_sig[i];
        const int off = t * dim32 + lane;
        if (hasZ) store_val(&(dzg + tok_blk)[off], e_gz[i] * yo);
        store_val(&(dxg + tok_blk)[off], gx);
        store_val(&(ddtg + tok_blk)[off], gdt);
        accD = fmaf(go, xv, accD);
        accBias += gdt;
      }
    }
    if (j > jbeg) {
      prologue(j - 1);
      if (j - 2 >= jbeg) gload(j - 2);
    }
  }

  // per-(segment, batch row) partial sums of dA, dD and dbias
  const int64_t prow = static_cast<int64_t>(seg) * sh.batch + b;
  if (dvalid) {
#pragma unroll
    for (int q = 0; q < S; ++q)
      if (n0 + q < N) gAp[(prow * N + n0 + q) * dim + d] = gA[q];
  }
  __syncthreads();
  s_r1[w][0][lane] = accD;
  s_r2[w][0][lane] = accBias;
  __syncthreads();
  if (w == 0 && dvalid) {
    float sD = 0.f, sb = 0.f;
#pragma unroll
    for (int q = 0; q < NW; ++q) {
      sD += s_r1[q][0][lane];
      sb += s_r2[q][0][lane];
    }
    gDp[prow * dim + d] = sD;
    gbp[prow * dim + d] = sb;
  }
}

// Reverse aggregates of the sequence split: for every segment but the last, the
// reverse recurrence G <- Abar (gyo C + G) run over the segment from G = 0 at its end
// gives the gradient its steps send to the state before its start (ragg_g); with the
// segment's sum of Delta*log2(e) (ragg_s), exp2(A * sum) is the product of Abar over
// it.  For N != 16 (N == 16 runs bwd_agg_row_kernel below): a workgroup per (batch
// row, channel tile, segment) with AS states per wave;
// blocks of kAggBlock steps staged through LDS, double-buffered so that the staging
// of the next block overlaps the steps of this one, with one barrier per block.
constexpr int kAggBlock = 32;

template <typename Tin, int NW, int AS, int NFIX>
__global__ __launch_bounds__(NW * 64) void bwd_agg_kernel(
    const Tin* __restrict__ dtg, const Tin* __restrict__ zg, const Tin* __restrict__ Cg,
    const Tin* __restrict__ dyg, const float* __restrict__ Ag, const float* __restrict__ biasg,
    float* __restrict__ ragg_g, float* __restrict__ ragg_s, BwdShape sh) {
  constexpr int T = kAggBlock;
  constexpr int NSP = NW * AS;   // states covered (N rounded up)
  constexpr int TPW = T / NW;
  static_assert(T % NW == 0, "block must split evenly over waves");
  static_assert(AS == 1 || AS == 2, "one or two states per wave");
  static_assert(T * NSP <= NW * 64, "one thread per staged C element");
  // (Delta * log2(e), gyo) of each staged timestep; C of each state (pairs for AS = 2)
  __shared__ float2 s_dg[2][T][kTile];
  __shared__ float s_C[2][T][NSP];
  __shared__ float s_sum[NW][kTile];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tid = threadIdx.x;
  // segments 1 .. nseg-1 (the first segment's aggregate is never needed)
  int64_t blk = xcd_remap(blockIdx.x, sh.ndtiles * sh.batch * (sh.nseg - 1));
  const int64_t dtile = blk % sh.ndtiles;
  blk /= sh.ndtiles;
  const int64_t b = blk % sh.batch;
  const int seg = static_cast<int>(blk / sh.batch) + 1;
  const int64_t L = sh.L, dim = sh.dim;
  const int N = NFIX > 0 ? NFIX : sh.N;
  const int dim32 = static_cast<int>(dim);
  const int64_t d = dtile * kTile + lane;
  const bool dvalid = d < dim;
  const int64_t dd = dvalid ? d : dim - 1;
  const bool hasZ = zg != nullptr;
  const float bias2 = biasg ? biasg[dd] * kLog2e : 0.f;
  // this wave's states n0 .. n0 + AS - 1; phantom states (n >= N) have A = 0, C = 0
  // and are not written
  const int n0 = AS * w;
  float An[AS], G[AS];
#pragma unroll
  for (int q = 0; q < AS; ++q) {
    An[q] = (n0 + q < N) ? Ag[dd * N + n0 + q] : 0.f;
    G[q] = 0.f;
  }
  float ssum = 0.f, scomp = 0.f;   // Kahan sum of this wave's staged Delta*log2(e)

  const int64_t l_beg = static_cast<int64_t>(seg) * sh.seg_blocks * kBwdBlock;
  const int64_t l_end = (l_beg + sh.seg_blocks * kBwdBlock < L) ? l_beg + sh.seg_blocks * kBwdBlock : L;
  const int64_t nb = (l_end - l_beg + T - 1) / T;
  const int64_t tok_b = b * L * dim + dtile * kTile;
  // inputs of one block, loaded one block ahead of their use
  Tin r_dt[TPW], r_z[TPW], r_dy[TPW];
  Tin r_c = Tin(0);
  const int c_t = tid / NSP, c_n = tid - (tid / NSP) * NSP;   // C element this thread stages
  const bool c_stager = tid < T * NSP;
  auto gload = [&](int64_t c) {
    const int64_t l0 = l_beg + c * T;
    const int cnt = static_cast<int>((l_end - l0) < T ? (l_end - l0) : T);
    const int64_t base = tok_b + l0 * dim;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = w + NW * i;
      Tin e = Tin(0), f = Tin(0), g = Tin(0);
      if (dvalid && t < cnt) {
        const int off = t * dim32 + lane;
        e = (dtg + base)[off];
        g = (dyg + base)[off];
        if (hasZ) f = (zg + base)[off];
      }
      r_dt[i] = e;
      r_z[i] = f;
      r_dy[i] = g;
    }
    r_c = (c_stager && c_n < N && c_t < cnt) ? Cg[(b * L + l0 + c_t) * N + c_n] : Tin(0);
  };
  auto prologue = [&](int64_t c, int buf) {
    const int64_t l0 = l_beg + c * T;
    const int cnt = static_cast<int>((l_end - l0) < T ? (l_end - l0) : T);
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = w + NW * i;
      const float zv = to_f32(r_z[i]), gy = to_f32(r_dy[i]);
      float go = gy;
      if (hasZ) go = gy * (zv * hw_rcp(1.f + hw_exp2(-zv * kLog2e)));
      const float d2 = (t < cnt) ? softplus_log2e(fmaf(to_f32(r_dt[i]), kLog2e, bias2)) : 0.f;
      s_dg[buf][t][lane] = make_float2(d2, go);
      const float yk = d2 - scomp;   // padded steps add 0
      const float tk = ssum + yk;
      scomp = (tk - ssum) - yk;
      ssum = tk;
    }
    if (c_stager) s_C[buf][c_t][c_n] = to_f32(r_c);
  };
  if (nb > 0) {
    gload(nb - 1);
    prologue(nb - 1, static_cast<int>((nb - 1) & 1));
    if (nb > 1) gload(nb - 2);
  }
  for (int64_t c = nb - 1; c >= 0; --c) {
    const int buf = static_cast<int>(c & 1);
    // block c is staged, and every wave is done with the other buffer (block c + 1)
    __syncthreads();
    if (c > 0) {
      prologue(c - 1, buf ^ 1);
      if (c > 1) gload(c - 2);
    }
#pragma unroll 8
    for (int t = T - 1; t >= 0; --t) {
      const float2 dg = s_dg[buf][t][lane];
#pragma unroll
      for (int q = 0; q < AS; ++q) G[q] = hw_exp2(dg.x * An[q]) * fmaf(dg.y, s_C[buf][t][n0 + q], G[q]);
    }
  }
  s_sum[w][lane] = ssum;
  __syncthreads();
  if (dvalid) {
    const int64_t row = (static_cast<int64_t>(seg) * sh.batch + b) * dim + d;
#pragma unroll
    for (int q = 0; q < AS; ++q)
      if (n0 + q < N) ragg_g[row * N + n0 + q] = G[q];
    if (w == 0) {
      float sum = 0.f;
#pragma unroll
      for (int q = 0; q < NW; ++q) sum += s_sum[q][lane];
      ragg_s[row] = sum;
    }
  }
}

// The same reverse aggregates for N == 16 with the forward's row layout: 16 waves,
// wave w owning channels 4w .. 4w+3 (one per 16-lane row) and lane n of a row owning
// state n.  Chunks of 16 steps are staged as above (wave w stages timestep w of the
// chunk, lane = channel) and consumed last chunk first.  Lane t of a row reads its
// channel's (Delta*log2(e), gyo) of timestep t once per chunk, and the DPP row
// broadcast hands timestep t's pair to the whole row, folded into the multiplies by A
// and by C; C of the lane's state comes as four 128-bit reads per chunk.  Per step and
// state: G <- exp2(Delta*log2(e) A) (gyo C + G), five VALU and no LDS access, against
// four VALU and two LDS reads with one state per wave.
template <typename Tin>
__global__ __launch_bounds__(1024) void bwd_agg_row_kernel(
    const Tin* __restrict__ dtg, const Tin* __restrict__ zg, const Tin* __restrict__ Cg,
    const Tin* __restrict__ dyg, const float* __restrict__ Ag, const float* __restrict__ biasg,
    float* __restrict__ ragg_g, float* __restrict__ ragg_s, BwdShape sh) {
  constexpr int T = 16, N = 16;
  constexpr int DP = kTile + 1;   // row stride 130 words: 2 mod 32
  constexpr int BR = T + 4;       // [state][timestep] rows of 20 words
  __shared__ float2 s_dg[2][T][DP];
  __shared__ __align__(16) float s_c[2][N][BR];
  __shared__ float s_sum[16][kTile];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 15, lr = lane >> 4;
  int64_t blk = xcd_remap(blockIdx.x, sh.ndtiles * sh.batch * (sh.nseg - 1));
  const int64_t dtile = blk % sh.ndtiles;
  blk /= sh.ndtiles;
  const int64_t b = blk % sh.batch;
  const int seg = static_cast<int>(blk / sh.batch) + 1;
  const int64_t L = sh.L, dim = sh.dim;
  // staging: lane = channel (clamped to an in-range one past dim)
  const int64_t d = dtile * kTile + lane;
  const bool dvalid = d < dim;
  const int64_t dd = dvalid ? d : dim - 1;
  const unsigned dlane = static_cast<unsigned>(dd - dtile * kTile) * sizeof(Tin);
  // recurrence: lane = (state ln, channel 4w + lr)
  const int cr = 4 * w + lr;
  const int64_t dr = dtile * kTile + cr;
  const bool drvalid = dr < dim;
  const int64_t drc = drvalid ? dr : dim - 1;
  const bool hasZ = zg != nullptr;
  const float bias2 = biasg ? biasg[dd] * kLog2e : 0.f;
  const float Av = Ag[drc * N + ln];

  const int64_t l_beg = static_cast<int64_t>(seg) * sh.seg_blocks * kBwdBlock;
  const int64_t l_end = (l_beg + sh.seg_blocks * kBwdBlock < L) ? l_beg + sh.seg_blocks * kBwdBlock : L;
  const int seg_n = static_cast<int>(l_end - l_beg);
  const int nch = (seg_n + T - 1) / T;
  const int64_t tok = (b * L + l_beg) * dim + dtile * kTile;
  const Tin* __restrict__ DTb = dtg + tok;
  const Tin* __restrict__ DYb = dyg + tok;
  const Tin* __restrict__ Zb = hasZ ? zg + tok : dtg + tok;
  // C staging: waves 0-7 stage rows 2w and 2w+1 of the chunk, lane j*16 + n state n
  // (waves 8-15 load the same rows and discard them)
  const bool cwave = w < 8;
  const int crow = 2 * (w & 7) + ((lane >> 4) & 1);
  const int cn = lane & 15;
  const Tin* __restrict__ Cs = Cg + (b * L + l_beg) * N;

  float G = 0.f;
  float ssum = 0.f, scomp = 0.f;   // Kahan sum of the staged Delta*log2(e) (lane = channel)
  // Two register sets of loaded inputs: a chunk's loads are issued two iterations
  // before it is staged, so that their latency is hidden behind two chunks of steps.
  Tin r_dt[2], r_z[2], r_dy[2], r_c[2];
  // Steady iterations (chunk c >= 4) load chunk c - 3, which is full, through running
  // offsets advanced by subtraction: run_ld = (c - 3) T dim, run_c = (c - 3) T N.
  const int64_t Tdim = static_cast<int64_t>(T) * dim, TN = static_cast<int64_t>(T) * N;
  const int64_t woff = static_cast<int64_t>(w) * dim, coff = static_cast<int64_t>(crow) * N + cn;
  int64_t run_ld = 0, run_c = 0;
  // loads of chunk c into set S; positions past the segment end read its last row
  // (those steps become identities in the staging)
  auto gload = [&](auto sc, auto steadyc, int c) {
    constexpr int S = decltype(sc)::value;
    constexpr bool STEADY = decltype(steadyc)::value;
    const int l = c * T + w;
    const int64_t off = STEADY ? run_ld + woff : static_cast<int64_t>(l < seg_n ? l : seg_n - 1) * dim;
    r_dt[S] = ld_off(DTb + off, dlane);
    r_dy[S] = ld_off(DYb + off, dlane);
    r_z[S] = ld_off(Zb + off, dlane);
    const int t = c * T + crow;
    r_c[S] = Cs[STEADY ? run_c + coff : static_cast<int64_t>(t < seg_n ? t : seg_n - 1) * N + cn];
  };
  // stage chunk c from register set S into LDS buffer P
  auto stage = [&](auto pc, auto sc, int c) {
    constexpr int P = decltype(pc)::value;
    constexpr int S = decltype(sc)::value;
    const bool lv = c * T + w < seg_n;
    const float gy = to_f32(r_dy[S]);
    const float go = hasZ ? gy * silu(to_f32(r_z[S])) : gy;
    const float d2 = lv ? softplus_log2e(fmaf(to_f32(r_dt[S]), kLog2e, bias2)) : 0.f;
    s_dg[P][w][lane] = make_float2(d2, lv ? go : 0.f);
    const float yk = d2 - scomp;   // padded steps add 0
    const float tk = ssum + yk;
    scomp = (tk - ssum) - yk;
    ssum = tk;
    // lanes that stage no C element store into their s_sum slot instead (written for
    // real only after the last chunk), so that no store here runs under a partial
    // exec mask near the DPP broadcasts
    float* cdst = (cwave && lane < 2 * N) ? &s_c[P][cn][crow] : &s_sum[w][lane];
    *cdst = (c * T + crow < seg_n) ? to_f32(r_c[S]) : 0.f;
  };
  // Processing step j handles chunk c = nch-1-j from LDS buffer j&1, stages chunk
  // c-1 (loaded into set (j+1)&1) into the other buffer and loads chunk c-3 into the
  // set just freed.  STEADY: c >= 3, so all of it exists and needs no branch.
  auto iteration = [&](auto pc, auto steadyc, int c) {
    constexpr int P = decltype(pc)::value;
    constexpr int Q = 1 - P;
    constexpr bool STEADY = decltype(steadyc)::value;
    const float2 sdg = s_dg[P][ln][cr];
    const float sd = sdg.x, sg = sdg.y;
    f32x4 cb[4];
    auto read_c = [&](int m) { cb[m] = *reinterpret_cast<const f32x4*>(&s_c[P][ln][4 * m]); };
    read_c(3);
    if (STEADY || c > 0) {
      stage(Par<Q>{}, Par<Q>{}, c - 1);
      if (STEADY || c > 2) gload(Par<Q>{}, steadyc, c - 3);
    }
    static_for<0, T>([&](auto ic) {
      constexpr int t = T - 1 - decltype(ic)::value;
      if constexpr (t == 15 || t == 12 || t == 9) {
        __builtin_amdgcn_sched_barrier(0);
        read_c((t - 9) / 3);
        __builtin_amdgcn_sched_barrier(0);
      }
      const float e = hw_exp2(row_bcast<t>(sd) * Av);
      const float gc = row_bcast<t>(sg) * cb[t >> 2][t & 3];
      G = e * (gc + G);
    });
    __syncthreads();
  };
  if (nch > 0) {
    gload(Par<0>{}, std::false_type{}, nch - 1);
    stage(Par<0>{}, Par<0>{}, nch - 1);
    if (nch > 1) gload(Par<1>{}, std::false_type{}, nch - 2);
    if (nch > 2) gload(Par<0>{}, std::false_type{}, nch - 3);
    __syncthreads();
    // buffer and register-set parities follow the processing order, so they stay
    // compile-time constants
    int c = nch - 1;
    run_ld = static_cast<int64_t>(c - 3) * Tdim;
    run_c = static_cast<int64_t>(c - 3) * TN;
    for (; c >= 4; c -= 2) {
      iteration(Par<0>{}, std::true_type{}, c);
      run_ld -= Tdim;
      run_c -= TN;
      iteration(Par<1>{}, std::true_type{}, c - 1);
      run_ld -= Tdim;
      run_c -= TN;
    }
    for (; c >= 1; c -= 2) {
      iteration(Par<0>{}, std::false_type{}, c);
      iteration(Par<1>{}, std::false_type{}, c - 1);
    }
    if (c == 0) iteration(Par<0>{}, std::false_type{}, 0);
  }
  s_sum[w][lane] = ssum;
  __syncthreads();
  const int64_t rowbase = static_cast<int64_t>(seg) * sh.batch + b;
  if (drvalid) ragg_g[(rowbase * dim + dr) * N + ln] = G;
  if (w == 0 && dvalid) {
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) sum += s_sum[q][lane];
    ragg_s[rowbase * dim + d] = sum;
  }
}

// gin[s] = gradient entering the end of segment s: gin[nseg-1] = dLoss/d(last state)
// (or 0), gin[s-1] = exp2(A * sum_s) * gin[s] + ragg_g[s].
__global__ __launch_bounds__(256) void bwd_carry_kernel(const float* __restrict__ ragg_g,
                                                        const float* __restrict__ ragg_s, const float* __restrict__ A,
                                                        const float* __restrict__ dlast, float* __restrict__ gin,
                                                        int64_t batch, int64_t dim, int N, int nseg) {
  const int64_t total = batch * dim * N;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t bd = i / N;
  const int n = static_cast<int>(i - bd * N);
  const int64_t d = bd % dim;
  const float a = A[d * N + n];
  float g = dlast ? dlast[i] : 0.f;
  // segments in groups of G, right to left: a group's aggregates are loaded together,
  // so their latencies overlap instead of adding up along the sequential combine
  constexpr int G = 8;
  for (int s0 = nseg - 1; s0 >= 0; s0 -= G) {
    float gv[G], sv[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int s = s0 - k;
      const bool have = s > 0;   // the first segment has no aggregate
      gv[k] = have ? ragg_g[static_cast<int64_t>(s) * total + i] : 0.f;
      sv[k] = have ? ragg_s[static_cast<int64_t>(s) * batch * dim + bd] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int s = s0 - k;
      if (s >= 0) {
        gin[static_cast<int64_t>(s) * total + i] = g;
        g = fmaf(hw_exp2(a * sv[k]), g, gv[k]);
      }
    }
  }
}

// The reductions after the reverse pass, in one launch.
//  * dB[b][l][n], dC[b][l][n] = sums over channel tiles of the partials (fixed order),
//    in the token dtype.  One thread per (b, n) and V consecutive l (V = 4 when L is a
//    multiple of 4: 16-byte partial loads), l fastest, so the partial reads coalesce;
//    the tiles are read in groups of G, whose loads are issued together and then added
//    in tile order (the same order as one at a time, so the sums are unchanged).
//  * dA[d][n], dD[d], dbias[d] = sums over (segment, batch row) partials (fixed order),
//    by the grid's last workgroups (from bc_blocks on): one thread per (n, d), d
//    fastest, so the partial reads ([row][n][dim]) coalesce.
template <typename Tin, int V>
__global__ __launch_bounds__(256) void bwd_reduce(const float* __restrict__ gBp, const float* __restrict__ gCp,
                                                  Tin* __restrict__ dB, Tin* __restrict__ dC, int64_t batch,
                                                  int64_t L, int N, int64_t ndtiles, unsigned bc_blocks,
                                                  const float* __restrict__ gAp, const float* __restrict__ gDp,
                                                  const float* __restrict__ gbp, float* __restrict__ dA,
                                                  float* __restrict__ dD, float* __restrict__ dbias, int64_t rows,
                                                  int64_t dim) {
  constexpr int G = 8;
  if (blockIdx.x >= bc_blocks) {
    const int64_t i = static_cast<int64_t>(blockIdx.x - bc_blocks) * blockDim.x + threadIdx.x;   // n * dim + d
    if (i >= dim * N) return;
    const int n = static_cast<int>(i / dim);
    const int64_t d = i - static_cast<int64_t>(n) * dim;
    float s = 0.f;
    for (int64_t r0 = 0; r0 < rows; r0 += G) {
      float v[G];
#pragma unroll
      for (int k = 0; k < G; ++k) v[k] = (r0 + k < rows) ? gAp[(r0 + k) * N * dim + i] : 0.f;
#pragma unroll
      for (int k = 0; k < G; ++k)
        if (r0 + k < rows) s += v[k];
    }
    dA[d * N + n] = s;
    if (n == 0) {
      float sD = 0.f, sb = 0.f;
      for (int64_t r0 = 0; r0 < rows; r0 += G) {
        float vD[G], vb[G];
#pragma unroll
        for (int k = 0; k < G; ++k) {
          vD[k] = (r0 + k < rows) ? gDp[(r0 + k) * dim + d] : 0.f;
          vb[k] = (r0 + k < rows) ? gbp[(r0 + k) * dim + d] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < G; ++k)
          if (r0 + k < rows) {
            sD += vD[k];
            sb += vb[k];
          }
      }
      if (dD) dD[d] = sD;
      if (dbias) dbias[d] = sb;
    }
    return;
  }
  const int64_t per_tile = batch * N * L;
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * V;   // (b * N + n) * L + l
  if (i >= per_tile) return;
  typedef float vec __attribute__((ext_vector_type(V)));
  vec sB = {}, sC = {};
  for (int64_t k0 = 0; k0 < ndtiles; k0 += G) {
    vec vb[G], vc[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
      if (k0 + k < ndtiles) {
        vb[k] = *reinterpret_cast<const vec*>(gBp + (k0 + k) * per_tile + i);
        vc[k] = *reinterpret_cast<const vec*>(gCp + (k0 + k) * per_tile + i);
      }
    }
#pragma unroll
    for (int k = 0; k < G; ++k)
      if (k0 + k < ndtiles) {
        sB += vb[k];
        sC += vc[k];
      }
  }
  const int64_t l = i % L;
  const int64_t bn = i / L;
  const int64_t n = bn % N, b = bn / N;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int64_t o = (b * L + l + v) * N + n;
    store_val(&dB[o], sB[v]);
    store_val(&dC[o], sC[v]);
  }
}

namespace {

template <typename Tin, int NW, int NF, bool EU>
void launch_bwd_one(const BwdParams& p, hipStream_t s) {
  BwdShape sh{p.batch, p.L, p.dim, p.ndtiles, p.nblk, p.seg_blocks, p.N, p.nseg};
  if (p.nseg > 1 && !p.carry_done) {   // else gin was formed by the checkpoint pass
    const dim3 agrid(static_cast<unsigned>(p.ndtiles * p.batch * (p.nseg - 1)));
    if (p.agg_done) {
      // the aggregates came from the checkpoint pass
    } else if constexpr (NF == 16) {
      hipLaunchKernelGGL((bwd_agg_row_kernel<Tin>), agrid, dim3(1024), 0, s, static_cast<const Tin*>(p.dt),
                         static_cast<const Tin*>(p.z), static_cast<const Tin*>(p.C), static_cast<const Tin*>(p.dy),
                         p.A, p.bias, p.ragg_g, p.ragg_s, sh);
    } else {
      // one state per wave in the aggregate pass: twice the reverse pass's waves, for
      // occupancy (measured: two states per wave was no faster on the training shape)
      constexpr int AS = 1;
      constexpr int AW = NW * kBwdSpw / AS;
      hipLaunchKernelGGL((bwd_agg_kernel<Tin, AW, AS, NF>), agrid, dim3(AW * 64), 0, s, static_cast<const Tin*>(p.dt),
                         static_cast<const Tin*>(p.z), static_cast<const Tin*>(p.C), static_cast<const Tin*>(p.dy),
                         p.A, p.bias, p.ragg_g, p.ragg_s, sh);
    }
    const int64_t total = p.batch * p.dim * p.N;
    hipLaunchKernelGGL(bwd_carry_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s,
                       p.ragg_g, p.ragg_s, p.A, p.dlast, p.gin, p.batch, p.dim, p.N, p.nseg);
  }
  hipLaunchKernelGGL((bwd_kernel<Tin, NW, NF, EU>), dim3(static_cast<unsigned>(p.ndtiles * p.batch * p.nseg)),
                     dim3(NW * 64), 0, s, static_cast<const Tin*>(p.x), static_cast<const Tin*>(p.dt),
                     static_cast<const Tin*>(p.z), static_cast<const Tin*>(p.B), static_cast<const Tin*>(p.C),
                     static_cast<const Tin*>(p.dy), p.A, p.Dskip, p.bias, p.dlast, p.nseg > 1 ? p.gin : nullptr,
                     p.ckpt, static_cast<Tin*>(p.dx), static_cast<Tin*>(p.ddt), static_cast<Tin*>(p.dz), p.gB_part,
                     p.gC_part, p.gA_part, p.gD_part, p.gbias_part, p.dh0, sh);
}

template <typename Tin, bool EU>
void launch_bwd_n(const BwdParams& p, hipStream_t s) {
  constexpr int WMAX = SSCAN_MAX_DSTATE / kBwdSpw;
  switch (bwd_waves(p.N)) {
    case 1: launch_bwd_one<Tin, 1, 0, EU>(p, s); break;
    case 2: launch_bwd_one<Tin, 2, 0, EU>(p, s); break;
    case 4: launch_bwd_one<Tin, 4, 0, EU>(p, s); break;
    default:
      if (p.N == 16)
        launch_bwd_one<Tin, WMAX, 16, EU>(p, s);
      else
        launch_bwd_one<Tin, WMAX, 0, EU>(p, s);
      break;
  }
}

template <typename Tin>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t s) {
  if (p.euler)
    launch_bwd_n<Tin, true>(p, s);
  else
    launch_bwd_n<Tin, false>(p, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nbl = p.batch * p.N * p.L;
  const int64_t ndn = p.dim * p.N;
  const unsigned params_blocks = static_cast<unsigned>((ndn + 255) / 256);
  if (p.L % 4 == 0) {
    const unsigned bc_blocks = static_cast<unsigned>((nbl / 4 + 255) / 256);
    hipLaunchKernelGGL((bwd_reduce<Tin, 4>), dim3(bc_blocks + params_blocks), dim3(256), 0, s, p.gB_part, p.gC_part,
                       static_cast<Tin*>(p.dB), static_cast<Tin*>(p.dC), p.batch, p.L, p.N, p.ndtiles, bc_blocks,
                       p.gA_part, p.gD_part, p.gbias_part, p.dA, p.dD, p.dbias, p.batch * p.nseg, p.dim);
  } else {
    const unsigned bc_blocks = static_cast<unsigned>((nbl + 255) / 256);
    hipLaunchKernelGGL((bwd_reduce<Tin, 1>), dim3(bc_blocks + params_blocks), dim3(256), 0, s, p.gB_part, p.gC_part,
                       static_cast<Tin*>(p.dB), static_cast<Tin*>(p.dC), p.batch, p.L, p.N, p.ndtiles, bc_blocks,
                       p.gA_part, p.gD_part, p.gbias_part, p.dA, p.dD, p.dbias, p.batch * p.nseg, p.dim);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, bool bf16, hipStream_t s) {
  if (p.batch <= 0 || p.dim <= 0) return hipSuccess;
  return bf16 ? launch_bwd_t<bf16_t>(p, s) : launch_bwd_t<float>(p, s);
}

}  // namespace sscan

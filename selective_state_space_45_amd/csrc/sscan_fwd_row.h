// Forward selective scan on gfx950, states across the lanes of a row.
//
// What is computed is the same as fwd_kernel's (velog.io Mamba review,
// "Discretization" and section 3.2; page-3 report sections 3 and 4.2): Delta =
// softplus(dt + bias), Abar = exp(Delta A), Bbar = (exp(Delta A) - 1)/A * B (or
// Delta B with the Euler rule), h_l = Abar h_{l-1} + Bbar x_l,
// y_l = (C_l . h_l + D x_l) * silu(z_l).
//
// Work decomposition.  A workgroup of 16 waves owns one (batch row, 64-channel tile,
// sequence segment).  Wave w owns channels 4w .. 4w+3 of the tile, one per 16-lane
// row of the wave, and lane n of a row owns state n (N <= 16; lanes past N hold a
// state that stays zero).  The sequence is consumed in chunks of 16 timesteps with one
// barrier per chunk:
//   prologue   wave w loads timestep w of the next chunk: x, dt, z coalesced along
//              channels (lane = channel), softplus and silu once per (l, d), and two
//              rows of B (waves 0-7) or C (waves 8-15); all of it staged to LDS.
//   recurrence (Delta*log2(e), x) of the chunk's timestep t for this lane's channel is
//              read once per chunk (lane n of a row reads timestep n, one 64-bit read)
//              and handed to every lane of the row by the DPP row broadcast
//              (row_newbcast:t) folded into the multiplies by A and by B, so the 16
//              steps need no further LDS reads for them.  B and C of the lane's state
//              for all 16 timesteps come from LDS as 128-bit reads (four each).
//   readout    each lane forms C_t h_t for its state; the sum over the 16 states of a
//              row is a reduce-scatter across the row's lanes (bank-masked DPP adds,
//              then quad permutes) that leaves lane t of the row holding y's C.h for
//              timestep t; one LDS store per lane then hands the chunk's 16 x 64 sums
//              to the epilogue.
//   epilogue   wave w adds D x, applies the gate and stores y of timestep w of the
//              previous chunk, coalesced along channels.
// Against fwd_kernel (one state per wave, lane = channel) this trades the per-step
// LDS traffic -- every wave reading every staged (Delta, x) and the N-way readout of
// states through LDS -- for DPP broadcasts and a register-only reduction; per wave and
// chunk the LDS traffic drops from ~16 KB to ~9 KB, most of it 128-bit reads of B and C.
// The state update is the same k-form: h <- Abar (h + k) - k with k = x B / A; a wave
// whose channels have some A == 0 takes the explicit form, as a wave-uniform branch.
#pragma once

#include "sscan_device.h"
#include "sscan_internal.h"
#include "sscan_lanes.h"

namespace sscan {

// Sum over the 16 lanes of each row of p[t], t = 0..15, scattered: lane t of the row
// ends with the row's sum for timestep t.  Four halvings; each pairs every lane with a
// partner in the other half of its group and keeps the half of the timesteps its own
// lane bit selects:
//   bit 3: partner lane ^ 8 (row_ror:8); lanes 0-7 keep t < 8.  Each output register
//          is written by two adds masked to lane groups of four (bank_mask), one per
//          half, so no selects are needed.
//   bit 2: partner lane ^ 7 within each half row (row_half_mirror); masked the same way.
//   bit 1, bit 0: partner lane ^ 2, ^ 1 (quad permutes); the kept and sent values are
//          chosen per lane with selects.
// The masked adds are written as inline assembly (the compiler has no masked-add
// builtin); each block starts with the two wait states that a DPP read of a VGPR
// written by the preceding VALU instruction requires.  All 64 lanes must be active.
__device__ __forceinline__ float row_reduce_scatter16(const float (&p)[16], int lane) {
  float q[8], r[4];
  asm("s_nop 1\n\t"
      "v_add_f32_dpp %0, %4, %4 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %0, %8, %8 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %1, %5, %5 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %1, %9, %9 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %2, %6, %6 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %2, %10, %10 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %3, %7, %7 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %3, %11, %11 row_ror:8 row_mask:0xf bank_mask:0xc"
      : "=&v"(q[0]), "=&v"(q[1]), "=&v"(q[2]), "=&v"(q[3])
      : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[8]), "v"(p[9]), "v"(p[10]), "v"(p[11]));
  asm("s_nop 1\n\t"
      "v_add_f32_dpp %0, %4, %4 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %0, %8, %8 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %1, %5, %5 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %1, %9, %9 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %2, %6, %6 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %2, %10, %10 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %3, %7, %7 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %3, %11, %11 row_ror:8 row_mask:0xf bank_mask:0xc"
      : "=&v"(q[4]), "=&v"(q[5]), "=&v"(q[6]), "=&v"(q[7])
      : "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7]), "v"(p[12]), "v"(p[13]), "v"(p[14]), "v"(p[15]));
  asm("s_nop 1\n\t"
      "v_add_f32_dpp %0, %4, %4 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %0, %8, %8 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %1, %5, %5 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %1, %9, %9 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %2, %6, %6 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %2, %10, %10 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %3, %7, %7 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %3, %11, %11 row_half_mirror row_mask:0xf bank_mask:0xa"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(q[4]), "v"(q[5]), "v"(q[6]), "v"(q[7]));
  const bool b1 = (lane & 2) != 0, b0 = (lane & 1) != 0;
  float s[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float keep = b1 ? r[j + 2] : r[j];
    const float send = b1 ? r[j] : r[j + 2];
    s[j] = keep + dpp_move<0x4E>(send);   // quad_perm [2,3,0,1]
  }
  const float keep = b0 ? s[1] : s[0];
  const float send = b0 ? s[0] : s[1];
  return keep + dpp_move<0xB1>(send);     // quad_perm [1,0,3,2]
}

// One workgroup: (batch row b, 64-channel tile, segment); 16 waves x 4 channels x 16
// states.  MODE: kFwdOut (y and the final state), kFwdCkpt (no y: the state entering
// every block of kBwdBlock steps, for the backward pass), kFwdOutCkpt (both),
// kFwdOutConv (kFwdOut on the output of the convolution prologue: x is the raw input
// of a causal depthwise conv1d over time, conv_w [dim][dconv] taps and optional
// conv_b [dim], followed by SiLU, as in the page-3 report's MambaBlock (section 3,
// forward); inputs before the sequence start come from conv_s [batch][dim][dconv-1],
// zeros when absent).
// NFIX: N as a compile-time constant (16) or 0 (from the shape, N <= 16).
template <typename Tin, int MODE, int NFIX, bool EULER>
__global__ __launch_bounds__(1024) void fwd_row_kernel(
    const Tin* __restrict__ xg, const Tin* __restrict__ dtg, const Tin* __restrict__ zg,
    const Tin* __restrict__ Bg, const Tin* __restrict__ Cg, const float* __restrict__ Ag,
    const float* __restrict__ Dg, const float* __restrict__ biasg, const float* __restrict__ h_init,
    Tin* __restrict__ yg, float* __restrict__ h_last, float* __restrict__ ckpt, const float* __restrict__ conv_w,
    const float* __restrict__ conv_b, const float* __restrict__ conv_s, FwdShape sh) {
  constexpr bool CONV = MODE == kFwdOutConv;
  constexpr bool OUT = MODE == kFwdOut || MODE == kFwdOutCkpt || CONV;
  constexpr bool CKPT = MODE == kFwdCkpt || MODE == kFwdOutCkpt;
  static_assert(MODE == kFwdOut || CKPT || CONV, "output, checkpoint and convolution modes");
  constexpr int T = kChunk;
  static_assert(T == 16, "one staged timestep per lane of a row");
  static_assert(!CKPT || 2 * kBwdBlock == T, "checkpoints are taken at half chunks");
  // LDS layouts.  Row strides are chosen so that each read below touches distinct
  // banks (16 lanes for 64-bit accesses, 32 for 32-bit ones, 8 for 128-bit ones).
  // (Delta*log2(e), x) [timestep][channel] (Delta*x for the Euler rule): the
  // recurrence reads timestep = lane's state index, hence a row stride of 130 words,
  // 2 mod 32.
  constexpr int DP = kTile + 1;
  // B and C: row = state, word = timestep; rows of 20 words keep 16-byte alignment
  // and spread 8 consecutive rows over all 32 banks.
  constexpr int BR = T + 4;
  constexpr int YP = kTile + 2;
  __shared__ float2 s_dx[2][T][DP];
  __shared__ __align__(16) float s_b[2][16][BR];
  __shared__ __align__(16) float s_c[OUT ? 2 : 1][16][BR];
  __shared__ float s_y[OUT ? 2 : 1][T][YP];
  // checkpoint states of a chunk's two blocks, [half][state][channel], so that they
  // leave as whole rows of 64 channels (the layout the backward pass reads)
  __shared__ float s_ck[CKPT ? 2 : 1][2][16][YP];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 15, lr = lane >> 4;

  int64_t blk = xcd_remap(blockIdx.x, sh.ndtiles * sh.batch * sh.nseg);
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
  const int nfull = seg_n / T;

  // prologue / epilogue: lane = channel (clamped to an in-range one past dim)
  const int64_t d = dtile * kTile + lane;
  const bool dvalid = d < dim;
  const int64_t dd = dvalid ? d : dim - 1;
  const unsigned dlane = static_cast<unsigned>(dd - dtile * kTile) * sizeof(Tin);
  // recurrence: lane = (state ln, channel 4w + lr)
  const int cr = 4 * w + lr;
  const int64_t dr = dtile * kTile + cr;
  const bool drvalid = dr < dim;
  const int64_t drc = drvalid ? dr : dim - 1;
  const bool nlive = ln < N;

  const int64_t tok0 = (b * L + l_begin) * dim + dtile * kTile;
  const Tin* __restrict__ Xb = xg + tok0;
  const Tin* __restrict__ DTb = dtg + tok0;
  const bool hasZ = OUT && zg != nullptr;
  const Tin* __restrict__ Zb = hasZ ? zg + tok0 : xg + tok0;
  Tin* __restrict__ Yb = OUT ? yg + tok0 : nullptr;
  // B/C staging loads: waves 0-7 load B, waves 8-15 load C (output modes), two rows
  // each; lane j*N + n loads state n of row j
  const Tin* __restrict__ BCs = ((w < 8 || !OUT) ? Bg : Cg) + (b * L + l_begin) * N;
  const bool bcwave = w < 8 || OUT;
  const int bcrow0 = 2 * (w & 7);
  const bool bclane = lane < 2 * N;
  const int bcj = bclane ? lane / N : 0;
  const int bcn = bclane ? lane - bcj * N : 0;
  const unsigned bcoff = static_cast<unsigned>(bclane ? lane : 0) * sizeof(Tin);

  const float bias2 = biasg ? biasg[dd] * kLog2e : 0.f;
  const float dsk = (OUT && Dg) ? Dg[dd] : 0.f;

  // A past N: any nonzero value; that state's B row is zero, so it stays zero.
  const float Av = nlive ? Ag[drc * N + ln] : -1.f;
  const float rA = (Av != 0.f) ? 1.f / Av : 0.f;
  const bool zeroA = __any(Av == 0.f);

  float h = 0.f;
  if (h_init && drvalid && nlive) h = h_init[((static_cast<int64_t>(seg) * sh.batch + b) * dim + dr) * N + ln];

  // CONV: taps and bias of this lane's channel; taps past dconv are zero
  constexpr int KC = CONV ? kMaxConv : 1;
  const int K = CONV ? sh.dconv : 1;
  float cw[KC];
  float cbias = 0.f;
  if constexpr (CONV) {
#pragma unroll
    for (int k = 0; k < KC; ++k) cw[k] = (k < K) ? conv_w[dd * K + k] : 0.f;
    cbias = conv_b ? conv_b[dd] : 0.f;
  }
  const Tin* __restrict__ Xrow = xg + b * L * dim + dtile * kTile;   // whole sequence of this row

  Tin rx, rdt, rz, rbc;
  Tin rxc[KC];
  // Global loads of chunk c for the prologue: x, dt, z of timestep w (lane = channel)
  // and this wave's B/C rows.  STEADY: chunk c is full.  Otherwise positions past the
  // segment end read its last row (those steps become identities in the prologue).
  auto gload = [&](auto steadyc, int c) {
    constexpr bool STEADY = decltype(steadyc)::value;
    const int l = c * T + w;
    const int64_t off = static_cast<int64_t>(STEADY ? l : (l < seg_n ? l : seg_n - 1)) * dim;
    if constexpr (CONV) {
      // raw inputs of the window l - (K-1) .. l, from positions clamped at the sequence
      // start (replaced from conv_s in the prologue); taps past K load position l
      const int64_t lg = l_begin + (STEADY ? l : (l < seg_n ? l : seg_n - 1));
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        const int back = (K - 1 - k) < 0 ? 0 : (K - 1 - k);
        const int64_t pos = lg - (back <= lg ? back : lg);
        rxc[k] = ld_off(Xrow + pos * dim, dlane);
      }
    } else {
      rx = ld_off(Xb + off, dlane);
    }
    rdt = ld_off(DTb + off, dlane);
    if constexpr (OUT) rz = ld_off(Zb + off, dlane);
    if (bcwave) {
      const int r0 = c * T + bcrow0;
      if constexpr (STEADY) {
        rbc = ld_off(BCs + static_cast<int64_t>(r0) * N, bcoff);
      } else {
        const int rr = r0 + bcj < seg_n ? r0 + bcj : seg_n - 1;
        rbc = ld_off(BCs + static_cast<int64_t>(rr) * N, static_cast<unsigned>(bcn) * sizeof(Tin));
      }
    }
  };
  float eg[2], ed[2];
  auto prologue = [&](auto pc, auto steadyc, int c) {
    constexpr int P = decltype(pc)::value;
    constexpr bool STEADY = decltype(steadyc)::value;
    float xv;
    if constexpr (CONV) {
      const int64_t l_glob = l_begin + c * T + w;
      float v[KC];
#pragma unroll
      for (int k = 0; k < KC; ++k) v[k] = to_f32(rxc[k]);
      if (l_glob < K - 1) {   // wave-uniform: the window reaches before the sequence
#pragma unroll
        for (int k = 0; k < KC; ++k) {
          const int64_t pos = l_glob - (K - 1) + k;
          if (pos < 0) v[k] = (conv_s && dvalid) ? conv_s[(b * dim + d) * (K - 1) + (K - 1) + pos] : 0.f;
        }
      }
      float acc = cbias;
#pragma unroll
      for (int k = 0; k < KC; ++k) acc = fmaf(cw[k], v[k], acc);
      xv = silu(acc);
    } else {
      xv = to_f32(rx);
    }
    float d2 = softplus_log2e(fmaf(to_f32(rdt), kLog2e, bias2));
    if constexpr (!STEADY) {   // a padded step is the identity: Delta = 0, x = 0
      const bool lv = c * T + w < seg_n;
      d2 = lv ? d2 : 0.f;
      xv = lv ? xv : 0.f;
    }
    s_dx[P][w][lane] = make_float2(d2, EULER ? (d2 * kLn2) * xv : xv);
    if (bcwave && bclane) {
      const int t = bcrow0 + bcj;
      if (w < 8)
        s_b[P][bcn][t] = to_f32(rbc);
      else if constexpr (OUT)
        s_c[P][bcn][t] = to_f32(rbc);
    }
    if constexpr (OUT) {
      if (hasZ)
        eg[P] = silu(to_f32(rz));
      else
        eg[P] = 1.f;
      ed[P] = dsk * xv;
    }
  };
  auto epilogue = [&](auto pc, int c, float g, float dx) {
    constexpr int P = decltype(pc)::value;
    if constexpr (OUT) {
      const int l = c * T + w;
      if (l < seg_n && dvalid) {
        const float v = s_y[P][w][lane];
        store_val(at_off(Yb + static_cast<int64_t>(l) * dim, static_cast<unsigned>(lane) * sizeof(Tin)), (v + dx) * g);
      }
    }
  };
  // Checkpoints: the state entering each half of chunk c goes to LDS during the steps;
  // after the chunk's barrier wave n stores row n of both halves, 64 channels
  // contiguous, to [batch][block][N][dim] (block = index of the kBwdBlock-step block).
  auto checkpoint = [&](auto pc, int half) {
    constexpr int P = decltype(pc)::value;
    if constexpr (CKPT) s_ck[P][half][ln][cr] = h;
  };
  auto ckpt_store = [&](auto pc, int c) {
    constexpr int P = decltype(pc)::value;
    if constexpr (CKPT) {
      if (w < N && dvalid) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int64_t kb = 2 * (l_begin / T + c) + half;
          if (kb < sh.nblk) ckpt[((b * sh.nblk + kb) * N + w) * dim + d] = s_ck[P][half][w][lane];
        }
      }
    }
  };

  auto iteration = [&](auto pc, auto steadyc, int c) {
    constexpr int P = decltype(pc)::value;
    constexpr int Q = 1 - P;
    constexpr bool STEADY = decltype(steadyc)::value;
    // (Delta*log2(e), x) of timestep ln for this lane's channel; B and C of its state
    const float2 sdx = s_dx[P][ln][cr];
    const float sd = sdx.x, sx = sdx.y;
    // B and C of group m (timesteps 4m .. 4m+3).  Group 0 is read here and the others
    // a few steps before they are needed (before steps 0, 3 and 6), each pinned in place
    // by a scheduling barrier: when all 16 waves issued their eight 128-bit reads at
    // the chunk start, the LDS issue queue filled and the waves stalled behind it
    // (training shape 0.399 ms with all reads up front, 0.374 spread out).
    f32x4 bb[4], cb[4];
    auto read_bc = [&](int m) {
      bb[m] = *reinterpret_cast<const f32x4*>(&s_b[P][ln][4 * m]);
      if constexpr (OUT) cb[m] = *reinterpret_cast<const f32x4*>(&s_c[P][ln][4 * m]);
    };
    read_bc(0);
    float pg = 0.f, pd = 0.f;
    if constexpr (OUT) {
      pg = eg[Q];
      pd = ed[Q];
    }
    if (STEADY || c + 1 < nchunks) {
      prologue(Par<Q>{}, steadyc, c + 1);
      if (STEADY || c + 2 < nchunks) gload(steadyc, c + 2);
    }
    if (STEADY || c >= 1) {
      epilogue(Par<Q>{}, c - 1, pg, pd);
      ckpt_store(Par<Q>{}, c - 1);
    }
    float p[T];
    if (EULER || !zeroA) {
      static_for<0, T>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        if constexpr (t == 0 || t == 3 || t == 6) {
          __builtin_amdgcn_sched_barrier(0);
          read_bc(t / 3 + 1);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (t % kBwdBlock == 0) checkpoint(pc, t / kBwdBlock);
        const float e = hw_exp2(row_bcast<t>(sd) * Av);
        const float xbt = row_bcast<t>(sx) * bb[t >> 2][t & 3];   // x_t B_t[n]
        if constexpr (EULER) {
          h = fmaf(e, h, xbt);
        } else {
          const float k = xbt * rA;
          h = fmaf(e, h + k, -k);
        }
        if constexpr (OUT) p[t] = cb[t >> 2][t & 3] * h;
      });
    } else {
      // some A == 0 among the wave's channels: h <- Abar h + g B x with
      // g = (Abar - 1)/A, or Delta where A == 0.  The broadcast is taken once, by
      // every lane, and both candidates are formed before the select: a DPP read
      // under a partial exec mask would see the inactive source lanes as zero.
      read_bc(1);
      read_bc(2);
      read_bc(3);
      static_for<0, T>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        if constexpr (t % kBwdBlock == 0) checkpoint(pc, t / kBwdBlock);
        const float dl2 = row_bcast<t>(sd);
        const float e = hw_exp2(dl2 * Av);
        const float gz = (e - 1.f) * rA, g0 = dl2 * kLn2;
        const float g = (Av != 0.f) ? gz : g0;
        h = fmaf(e, h, g * (row_bcast<t>(sx) * bb[t >> 2][t & 3]));
        if constexpr (OUT) p[t] = cb[t >> 2][t & 3] * h;
      });
    }
    if constexpr (OUT) s_y[P][ln][cr] = row_reduce_scatter16(p, lane);
    __syncthreads();
  };

  // zero once: the B/C rows of states past N (never written afterwards)
  for (int i = threadIdx.x; i < 2 * 16 * BR; i += 1024) {
    (&s_b[0][0][0])[i] = 0.f;
    if constexpr (OUT) (&s_c[0][0][0])[i] = 0.f;
  }
  __syncthreads();
  if (nchunks > 0) {
    gload(std::false_type{}, 0);
    prologue(Par<0>{}, std::false_type{}, 0);
    if (nchunks > 1) gload(std::false_type{}, 1);
    __syncthreads();
    iteration(Par<0>{}, std::false_type{}, 0);
    // steady iterations: c >= 1 and chunks c + 1, c + 2 full (pairs, so the LDS
    // buffer index stays a compile-time constant)
    int c = 1;
    for (; c + 3 < nfull; c += 2) {
      iteration(Par<1>{}, std::true_type{}, c);
      iteration(Par<0>{}, std::true_type{}, c + 1);
    }
    for (; c < nchunks; c += 2) {
      iteration(Par<1>{}, std::false_type{}, c);
      if (c + 1 < nchunks) iteration(Par<0>{}, std::false_type{}, c + 1);
    }
    if ((nchunks - 1) & 1) {
      epilogue(Par<1>{}, nchunks - 1, eg[1], ed[1]);
      ckpt_store(Par<1>{}, nchunks - 1);
    } else {
      epilogue(Par<0>{}, nchunks - 1, eg[0], ed[0]);
      ckpt_store(Par<0>{}, nchunks - 1);
    }
  }
  if constexpr (OUT) {
    if (h_last && seg == sh.nseg - 1 && drvalid && nlive) h_last[(b * dim + dr) * N + ln] = h;
  }
}

template <typename Tin, int MODE, int NF, bool EU>
void launch_row_one(const FwdParams& p, dim3 grid, hipStream_t s) {
  FwdShape sh{p.batch, p.L, p.dim, p.seg_len, p.ndtiles, p.nblk, p.N, p.nseg, p.dconv};
  hipLaunchKernelGGL((fwd_row_kernel<Tin, MODE, NF, EU>), grid, dim3(1024), 0, s, static_cast<const Tin*>(p.x),
                     static_cast<const Tin*>(p.dt), static_cast<const Tin*>(p.z), static_cast<const Tin*>(p.B),
                     static_cast<const Tin*>(p.C), p.A, p.Dskip, p.bias, p.h_init, static_cast<Tin*>(p.y), p.h_last,
                     p.ckpt, p.conv_w, p.conv_b, p.conv_s, sh);
}

// Launch of one (mode, discretization rule) variant of the row layout (N <= 16).
template <int MODE, bool EU>
hipError_t launch_fwd_row(const FwdParams& p, bool bf16, hipStream_t s) {
  const int64_t nblocks = p.ndtiles * p.batch * p.nseg;
  if (nblocks <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(nblocks));
  if (bf16) {
    if (p.N == 16)
      launch_row_one<bf16_t, MODE, 16, EU>(p, grid, s);
    else
      launch_row_one<bf16_t, MODE, 0, EU>(p, grid, s);
  } else {
    if (p.N == 16)
      launch_row_one<float, MODE, 16, EU>(p, grid, s);
    else
      launch_row_one<float, MODE, 0, EU>(p, grid, s);
  }
  return hipGetLastError();
}

}  // namespace sscan

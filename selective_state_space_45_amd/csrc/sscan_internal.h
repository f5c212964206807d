// Internal interface between the C entry points (sscan_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sscan {

constexpr int kTile = 64;     // channels per workgroup: one per lane of a wave
constexpr int kChunk = 16;    // timesteps staged through LDS per chunk
constexpr int kBwdBlock = 8;  // timesteps per backward block = checkpoint spacing
constexpr int kMaxConv = 4;   // taps of the fused convolution prologue (Mamba's d_conv)

// Modes of the forward kernel.
constexpr int kFwdOut = 0;    // y (and the final state)
constexpr int kFwdAgg = 1;    // per-segment aggregates for the two-level scan
constexpr int kFwdCkpt = 2;   // states entering every kBwdBlock steps, for the backward pass
constexpr int kFwdOutCkpt = 3;  // y and the final state, and the kFwdCkpt states as well
constexpr int kFwdOutConv = 4;  // kFwdOut with the convolution prologue (row layout only)
constexpr int kFwdCkptAgg = 5;  // kFwdCkpt, and the backward pass's segment carries for two
                                // reverse segments (row layout, N == 16, one forward segment)

struct FwdParams {
  const void* x;
  const void* dt;
  const void* z;          // nullable
  const void* B;
  const void* C;
  const float* A;         // [dim][N]
  const float* Dskip;     // nullable
  const float* bias;      // nullable
  const float* h_init;    // [nseg or 1][batch][dim][N] or null: state entering each segment
  void* y;
  float* h_last;          // nullable, written by the last segment
  float* agg_h;           // aggregate pass: [nseg][batch][dim][N] local end state
  float* agg_s;           // aggregate pass: [nseg][batch][dim]    sum of Delta*log2(e)
  float* ckpt;            // checkpoint pass: [batch][nblk][N][dim] state entering each block
  int64_t nblk;           // backward blocks over the whole sequence: ceil(L / kBwdBlock)
  const float* conv_w;    // convolution prologue (nullable): taps [dim][dconv]
  const float* conv_b;    // nullable: [dim]
  const float* conv_s;    // nullable: raw inputs before the sequence [batch][dim][dconv-1]
  int dconv;
  // kFwdCkptAgg: the output gradient and dLoss/d(last state) (nullable), and either
  //  - rseg_len > 0: the backward pass's gin [2][batch][dim][N] (as its carry kernel
  //    forms it) for two reverse segments, the second starting at rseg_len (a multiple
  //    of kChunk below L), one forward segment; or
  //  - rseg_len == 0: the reverse aggregate of each forward segment, which is also a
  //    reverse segment, into gin as [nseg][batch][dim][N] and its sum of
  //    Delta*log2(e) into ragg_s [nseg][batch][dim] (what the backward pass's
  //    aggregate kernel writes; its carry kernel then chains them).
  const void* dy;
  const float* dlast;
  float* gin;
  float* ragg_s;
  int64_t rseg_len;
  int64_t batch, L, dim;
  int64_t seg_len;        // timesteps per segment (multiple of kChunk unless nseg == 1)
  int64_t ndtiles;        // ceil(dim / kTile)
  int N;
  int nseg;
  int npw;                // states per wave: 1, or 2 (N >= 3; the output mode then stages one
                          // C.h partial per wave, and two workgroups share a CU)
  bool euler;             // Bbar = Delta * B instead of the zero-order hold
  bool structured;        // the caller states A[d, n] = c_d a_n (SSCAN_FLAG_STRUCTURED_A)
};

// Sizes passed by value to the forward kernels (pointers go as separate
// restrict-qualified arguments so the compiler can keep B/C loads scalar).
struct FwdShape {
  int64_t batch, L, dim, seg_len, ndtiles, nblk, rseg_len;
  int N, nseg, dconv;
};

struct StepParams {
  float* state;
  const void* x;
  const void* dt;
  const void* z;
  const void* B;
  const void* C;
  const float* A;
  const float* Dskip;
  const float* bias;
  void* y;
  float* conv_state;      // convolution prologue (nullable): [batch][dim][dconv-1], in-out
  const float* conv_w;    // [dim][dconv]
  const float* conv_b;    // nullable: [dim]
  int64_t batch, dim;
  int N;
  int dconv;
  bool euler;             // Bbar = Delta * B instead of the zero-order hold
};

// Backward pass.  Workspace regions are carved by the host (sscan_api.hip).
struct BwdParams {
  const void* x;
  const void* dt;
  const void* z;          // nullable
  const void* B;
  const void* C;
  const void* dy;
  const float* A;
  const float* Dskip;     // nullable
  const float* bias;      // nullable
  const float* dlast;     // nullable: dLoss / d(last state) [batch][dim][N]
  const float* ckpt;      // [batch][nblk][N][dim] state entering each block of kBwdBlock steps
  void* dx;
  void* ddt;
  void* dz;               // nullable (iff z is)
  float* gB_part;         // [ndtiles][batch][N][L] per channel-tile partial sums
  float* gC_part;         // [ndtiles][batch][N][L]
  float* gA_part;         // [nseg][batch][N][dim]
  float* gD_part;         // [nseg][batch][dim]
  float* gbias_part;      // [nseg][batch][dim]
  float* dh0;             // nullable: [batch][dim][N]
  void* dB;               // [batch][L][N] (token dtype)
  void* dC;
  float* dA;              // [dim][N]
  float* dD;              // nullable
  float* dbias;           // nullable
  // sequence split of the reverse pass (nseg > 1): per-segment aggregates and carries
  float* ragg_g;          // [nseg][batch][dim][N] gradient leaving each segment's start from a zero end
  float* ragg_s;          // [nseg][batch][dim]    sum of Delta*log2(e) over each segment
  float* gin;             // [nseg][batch][dim][N] gradient entering each segment's end
  int64_t batch, L, dim, ndtiles, nblk;
  int64_t seg_blocks;     // blocks of kBwdBlock steps per segment
  int N;
  int nseg;
  bool euler;
  bool carry_done;        // gin already written (by the kFwdCkptAgg checkpoint pass)
  bool agg_done;          // ragg_g / ragg_s already written (by the kFwdCkptAgg checkpoint
                          // pass with per-segment aggregates); the carry kernel still runs
};

struct BwdShape {
  int64_t batch, L, dim, ndtiles, nblk, seg_blocks;
  int N, nseg;
};

hipError_t launch_bwd(const BwdParams& p, bool bf16, hipStream_t s);

// Waves per workgroup of the forward kernel with npw states per wave.
int fwd_nsplit(int npw, int N);
// Whether a forward launch takes the row layout (fwd_row_kernel).
bool fwd_row_layout(const FwdParams& p);

// Launchers; return hipSuccess or the launch error.
hipError_t launch_fwd_main(const FwdParams& p, bool bf16, hipStream_t s);
hipError_t launch_fwd_aggregate(const FwdParams& p, bool bf16, hipStream_t s);
hipError_t launch_fwd_checkpoints(const FwdParams& p, bool bf16, hipStream_t s);
// kFwdCkptAgg: N == 16, nseg == 1, rseg_len a positive multiple of kChunk below L
hipError_t launch_fwd_checkpoints_agg(const FwdParams& p, bool bf16, hipStream_t s);
hipError_t launch_fwd_carry(const float* agg_h, const float* agg_s, const float* A, const float* h_init,
                            float* carry, int64_t batch, int64_t dim, int N, int nseg, hipStream_t s);
hipError_t launch_fill_state(float* dst, const float* src, int64_t n, hipStream_t s);
// Convolution state after a sequence: the last dconv - 1 raw inputs (from x, or the
// incoming state when seqlen < dconv - 1); out may equal in.
hipError_t launch_conv_state(const void* x, const float* in, float* out, int64_t batch, int64_t L, int64_t dim,
                             int dconv, bool bf16, hipStream_t s);
hipError_t launch_step(const StepParams& p, bool bf16, hipStream_t s);

}  // namespace sscan

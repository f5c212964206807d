// Internal interface between the C entry points (sscan_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sscan {

constexpr int kTile = 64;     // channels per workgroup: one per lane of a wave
constexpr int kChunk = 16;    // timesteps staged through LDS per chunk

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
  int64_t batch, L, dim;
  int64_t seg_len;        // timesteps per segment (multiple of kChunk unless nseg == 1)
  int64_t ndtiles;        // ceil(dim / kTile)
  int N;
  int nseg;
  bool euler;             // Bbar = Delta * B instead of the zero-order hold
};

// Sizes passed by value to the forward kernels (pointers go as separate
// restrict-qualified arguments so the compiler can keep B/C loads scalar).
struct FwdShape {
  int64_t batch, L, dim, seg_len, ndtiles;
  int N, nseg;
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
  int64_t batch, dim;
  int N;
  bool euler;             // Bbar = Delta * B instead of the zero-order hold
};

// Waves per workgroup of the forward kernels for a given N (each wave owns one state).
int fwd_nsplit(int N);

// Launchers; return hipSuccess or the launch error.
hipError_t launch_fwd_main(const FwdParams& p, bool bf16, hipStream_t s);
hipError_t launch_fwd_aggregate(const FwdParams& p, bool bf16, hipStream_t s);
hipError_t launch_fwd_carry(const float* agg_h, const float* agg_s, const float* A, const float* h_init,
                            float* carry, int64_t batch, int64_t dim, int N, int nseg, hipStream_t s);
hipError_t launch_fill_state(float* dst, const float* src, int64_t n, hipStream_t s);
hipError_t launch_step(const StepParams& p, bool bf16, hipStream_t s);

}  // namespace sscan

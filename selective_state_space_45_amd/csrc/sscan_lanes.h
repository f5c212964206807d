// Cross-lane and addressing helpers shared by the row-layout kernels (gfx950):
// compile-time loops, DPP row broadcasts and moves, 32-bit-offset global accesses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sscan {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Compile-time loop: f(integral_constant<I>) for I = B .. E-1.
template <int I, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < E) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, E>(f);
  }
}

// Lane T's value of each 16-lane row, broadcast to the row (DPP row_newbcast, gfx90a
// and later).  Used as an operand, it folds into the consuming instruction.
template <int T>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + T, 0xf, 0xf, true));
}
// Full-row DPP move with control word CTRL (quad permutes here).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}

// 32-bit byte offsets from a wave-uniform base, so that global accesses use a scalar
// base plus a 32-bit vector offset.
template <typename Tp>
__device__ __forceinline__ Tp ld_off(const Tp* __restrict__ base, unsigned byte_off) {
  return *reinterpret_cast<const Tp*>(reinterpret_cast<const char*>(base) + byte_off);
}
template <typename Tp>
__device__ __forceinline__ Tp* at_off(Tp* base, unsigned byte_off) {
  return reinterpret_cast<Tp*>(reinterpret_cast<char*>(base) + byte_off);
}

}  // namespace sscan

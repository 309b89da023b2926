// Cross-lane helpers for 64-wide waves (DPP row operations + readlane).
#pragma once

#include <hip/hip_runtime.h>

namespace kvq {

// DPP controls (gfx9 encoding)
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- 7 - i within 8
constexpr int kDppMirror = 0x140;      // lane i <- 15 - i within 16
constexpr int kDppRor(int n) { return 0x120 + n; }  // rotate right by n within 16

// Every control used here reads a valid lane, so bound_ctrl does not change the result;
// this form lets the compiler fold the move into the consuming op (v_add_f32_dpp).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}

__device__ __forceinline__ float readlane(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// Sum over aligned groups of N consecutive lanes (N = 1, 2, 4, 8, 16); every lane of
// the group gets the total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<kDppXor1>(x);
  if constexpr (N >= 4) x += dpp<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppMirror>(x);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  x = fmaxf(x, dpp<kDppHalfMirror>(x));
  x = fmaxf(x, dpp<kDppMirror>(x));
  return fmaxf(fmaxf(readlane(x, 0), readlane(x, 16)), fmaxf(readlane(x, 32), readlane(x, 48)));
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  x += dpp<kDppMirror>(x);
  return (readlane(x, 0) + readlane(x, 16)) + (readlane(x, 32) + readlane(x, 48));
}

// Sum over the lanes that share (lane % N), N = 1, 2, 4, 8, 16 (strided groups).
template <int N>
__device__ __forceinline__ float strided_sum(float x) {
  if constexpr (N <= 1) x += dpp<kDppRor(1)>(x);
  if constexpr (N <= 2) x += dpp<kDppRor(2)>(x);
  if constexpr (N <= 4) x += dpp<kDppRor(4)>(x);
  if constexpr (N <= 8) x += dpp<kDppRor(8)>(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Order LDS traffic between the lanes of one wave (no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace kvq

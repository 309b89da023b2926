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

// Maximum over the wave, for values that are never NaN: max with DPP operands inside
// each row of 16 lanes, then the row broadcasts carry rows 0-2 into row 3, and lane 63
// holds the result.  (Written out because the compiler keeps a canonicalizing copy
// around every max of a DPP-moved value.)  Each DPP read of a register written by the
// previous VALU op needs two wait states, hence the s_nop 1 before it.
__device__ __forceinline__ float wave_max(float x) {
  asm("s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf"
      : "+v"(x));
  return readlane(x, 63);
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  x += dpp<kDppMirror>(x);
  return (readlane(x, 0) + readlane(x, 16)) + (readlane(x, 32) + readlane(x, 48));
}

// Reduce-scatter over the lanes that share lane % LPT (LPT = 2, 4, 8, 16): every lane
// brings V values, and afterwards v[0 .. V * LPT / 64) of lane l hold sums over its
// 64 / LPT lanes, of the original indices reduce_scatter_first<LPT, V>(l) + i.  Each step
// halves the values a lane keeps: at distance DIST (32, 16, ..., LPT) the lane keeps the
// lower half if (lane & DIST) == 0, else the upper half, and adds its partner's copy of it.
// The two cross-row steps are one v_permlane32_swap / v_permlane16_swap per pair (the swap
// trades the upper 32 lanes (odd rows) of the first operand for the lower 32 lanes (even
// rows) of the second), the steps inside a row a DPP or swizzle move.
template <int DIST>
__device__ __forceinline__ float fold_pair(float x, float y, int lane) {
  if constexpr (DIST == 32 || DIST == 16) {
    const auto r = DIST == 32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false)
                              : __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    // lanes with (lane & DIST) == 0: own x + partner's x; the others: partner's y + own y
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    const bool hi = lane & DIST;
    const float keep = hi ? y : x, send = hi ? x : y;
    float got;
    if constexpr (DIST == 8) got = dpp<kDppRor(8)>(send);          // rotating a row by 8 pairs l with l ^ 8
    else if constexpr (DIST == 2) got = dpp<kDppXor2>(send);
    else got = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(send), 0x1F | (DIST << 10)));  // bit mode: l ^ DIST
    return keep + got;
  }
}

template <int DIST, int LPT, int N, int V>
__device__ __forceinline__ void reduce_scatter_step(float (&v)[V], int lane) {
  if constexpr (DIST >= LPT) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) v[i] = fold_pair<DIST>(v[i], v[i + N / 2], lane);
    reduce_scatter_step<DIST / 2, LPT, N / 2>(v, lane);
  }
}

template <int LPT, int V>
__device__ __forceinline__ void reduce_scatter(float (&v)[V], int lane) {
  static_assert(LPT >= 2 && LPT <= 16 && V * LPT % 64 == 0, "reduce_scatter shape");
  reduce_scatter_step<32, LPT, V>(v, lane);
}

template <int LPT, int V>
__device__ __forceinline__ int reduce_scatter_first(int lane) {
  int first = 0, n = V;
#pragma unroll
  for (int dist = 32; dist >= LPT; dist /= 2, n /= 2)
    if (lane & dist) first += n / 2;
  return first;
}

// Order LDS traffic between the lanes of one wave (no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace kvq

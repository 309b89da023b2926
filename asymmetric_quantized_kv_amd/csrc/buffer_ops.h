// Raw buffer loads for 64-wide waves: a buffer resource over a byte range, loaded through
// with a per-lane 32-bit offset and a wave-uniform offset, so that addresses cost no vector
// ALU.  A load past the resource's size returns 0 and touches no memory.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace kvq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint8_t* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), 0, (int)bytes, 0x00020000);
}

// W dwords at byte voff + soff: 16-byte loads for W a multiple of 4, else one 8- or 4-byte load
template <int W>
__device__ __forceinline__ void buf_dwords(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t (&o)[W]) {
  if constexpr (W % 4 == 0) {
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(voff + 16 * i), (int)soff, 0);
      o[4 * i] = t.x; o[4 * i + 1] = t.y; o[4 * i + 2] = t.z; o[4 * i + 3] = t.w;
    }
  } else if constexpr (W == 2) {
    const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0);
    o[0] = t.x; o[1] = t.y;
  } else {
    static_assert(W == 1, "dword count");
    o[0] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
  }
}

__device__ __forceinline__ uint16_t buf_u16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
}

__device__ __forceinline__ uint16_t buf_u8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0);
}

}  // namespace kvq

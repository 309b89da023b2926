// Quantize-on-append: new tokens' keys and values are encoded block by block and
// written at the end of the session cache ("KVSplit -- contexto 2 a 3 vezes mais longo
// em Apple Silicon", section "Opinioes no Hacker News": the cache is quantized at run
// time as tokens are processed; bit widths per "Principais resultados de benchmark").
//
// Four lanes own one 32-element block (8 elements each): loads and stores of a wave are
// contiguous and 8 to 32 bytes wide per lane, the block's amax is reduced over the 4 lanes
// with two DPP steps, and every lane encodes its own 8 elements.  Rounding follows the
// format fixed in include/kvq.h: fp32 IEEE division, fp16 round-to-nearest-even for the
// scale, round-half-away for the codes.
// fp8 keys (OCP MX blocks: a power-of-two block scale and E4M3 codes, the FP8
// alternative of "KV Cache Offloading for Context-Intensive Tasks", section
// "2. Metodologia") take the exponent from the amax's fp32 bits; the division by a
// power of two is exact and the E4M3 rounding is done in fp32 integer steps.
#include "kvq_internal.h"
#include "wave_ops.h"

namespace kvq {
namespace {

template <int DT>
__device__ __forceinline__ void load8(const void* src, int64_t elem, float (&x)[8]) {
  if constexpr (DT == 0) {  // fp32
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(src) + elem);
    const float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  } else {
    const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + elem);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t b = (w[i / 2] >> (16 * (i & 1))) & 0xffffu;
      if constexpr (DT == 1) {  // bf16: the upper half of an fp32
        x[i] = __uint_as_float(b << 16);
      } else {                  // fp16
        x[i] = (float)__builtin_bit_cast(_Float16, (uint16_t)b);
      }
    }
  }
}

// maximum over the 4 lanes of an aligned quad (values are never NaN here)
__device__ __forceinline__ float quad_max(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  return fmaxf(x, dpp<kDppXor2>(x));
}

__device__ __forceinline__ uint16_t f16_bits(float x) {
  _Float16 h = (_Float16)x;  // round to nearest even
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}

// E4M3 code of an exact fp32 value y: nearest, ties to even, saturated at +-448, +0 for 0.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const float a = fabsf(y);
  uint32_t c;
  if (a >= 448.f) {
    c = 0x7E;
  } else if (a < 0.015625f) {                       // below 2^-6: multiples of 2^-9
    c = (uint32_t)rintf(a * 512.f);                 // 8 lands on 2^-6, code 0x08
  } else {
    int ex = (int)((__float_as_uint(a) >> 23) & 255) - 127;             // -6 .. 8
    const float up = __uint_as_float((uint32_t)(127 + 3 - ex) << 23);   // 2^(3 - ex)
    uint32_t mm = (uint32_t)rintf(a * up);          // 8 .. 16, exact product
    if (mm == 16) { ++ex; mm = 8; }
    c = ((uint32_t)(ex + 7) << 3) | (mm - 8);
    if (c == 0x7F) c = 0x7E;                        // 480 is not a number in E4M3
  }
  return (y < 0.f && c != 0) ? (c | 0x80u) : c;
}

template <int BITS, int DT, int D>
__device__ __forceinline__ void encode_one(const void* src, uint8_t* region, int64_t row, int64_t elem, int blk,
                                           int sub, int64_t code_off, int64_t scale_off, int code_row,
                                           int scale_row) {
  float x[8];
  load8<DT>(src, elem, x);
  uint8_t* codes = region + code_off + row * code_row;
  float amax = 0.f;
  if constexpr (BITS != 16) {
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = quad_max(amax);
  }
  if constexpr (BITS == 16) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = f16_bits(x[2 * i]) | ((uint32_t)f16_bits(x[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(codes + (blk * 32 + sub * 8) * 2) = make_uint4(w[0], w[1], w[2], w[3]);
  } else if constexpr (BITS == kF8) {
    // e = floor(log2 amax) - 8 (the exponent of E4M3's largest binade), in [-127, 127];
    // a zero or subnormal amax gives -127
    const int eb = (int)((__float_as_uint(amax) >> 23) & 255);
    const int e = eb == 0 ? -127 : max(eb - 127 - 8, -127);
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);       // 2^-e, normal
    uint32_t w[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i / 4] |= e4m3_code(x[i] * inv) << (8 * (i & 3));
    *reinterpret_cast<uint2*>(codes + blk * 32 + sub * 8) = make_uint2(w[0], w[1]);
    if (sub == 0) region[scale_off + row * scale_row + blk] = (uint8_t)(e + 127);
  } else {
    constexpr float qmax = BITS == 8 ? 127.f : 7.f;
    const float d32 = fminf(amax / qmax, 65504.f);       // IEEE division, saturate
    const _Float16 d16 = (_Float16)d32;                   // round to nearest even
    const float d = (float)d16;
    int q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float y = d != 0.f ? x[i] / d : 0.f;          // IEEE division
      const float r = fminf(fmaxf(roundf(y), -qmax), qmax);   // half away from zero, clamp
      q[i] = (int)r;
    }
    if constexpr (BITS == 8) {
      uint32_t w[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
        w[h] = (q[4 * h] & 0xff) | ((q[4 * h + 1] & 0xff) << 8) | ((q[4 * h + 2] & 0xff) << 16) |
               ((uint32_t)(q[4 * h + 3] & 0xff) << 24);
      *reinterpret_cast<uint2*>(codes + blk * 32 + sub * 8) = make_uint2(w[0], w[1]);
    } else {
      uint32_t w = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) w |= (uint32_t)(q[i] + 8) << (4 * i);
      *reinterpret_cast<uint32_t*>(codes + blk * 16 + sub * 4) = w;
    }
    if (sub == 0) *reinterpret_cast<uint16_t*>(region + scale_off + row * scale_row + blk * 2) = __builtin_bit_cast(uint16_t, d16);
  }
}

template <int KB, int VB, int DT, int D>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int kNb = D / kBlock;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = a.n * a.hkv * kNb * 4;
  if (tid >= total) return;       // whole 4-lane groups drop out together (total % 4 == 0)
  const int sub = (int)(tid & 3);
  const int64_t bidx = tid >> 2;  // (token, head, block)
  const int blk = (int)(bidx % kNb);
  const int64_t th = bidx / kNb;  // token * hkv + head
  const int head = (int)(th % a.hkv);
  const int64_t tok = th / a.hkv;
  const int64_t elem = th * D + blk * kBlock + sub * 8;
  const int64_t row = a.t0 + tok;
  uint8_t* region = a.layer_base + (int64_t)head * a.g.region();
  if (blockIdx.y == 0)
    encode_one<KB, DT, D>(a.src[0], region, row, elem, blk, sub, a.g.off_kc(), a.g.off_ks(), a.g.kc, a.g.ks);
  else
    encode_one<VB, DT, D>(a.src[1], region, row, elem, blk, sub, a.g.off_vc(), a.g.off_vs(), a.g.vc, a.g.vs);
}

template <int KB, int VB, int DT, int D>
hipError_t launch_t(const AppendArgs& a, hipStream_t s) {
  const int64_t total = a.n * a.hkv * (D / kBlock) * 4;
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((append_kernel<KB, VB, DT, D>), dim3((unsigned)blocks, 2), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int KB, int VB, int DT>
hipError_t launch_d(const AppendArgs& a, int d, hipStream_t s) {
  if (d == 64) return launch_t<KB, VB, DT, 64>(a, s);
  if (d == 128) return launch_t<KB, VB, DT, 128>(a, s);
  return hipErrorInvalidValue;
}

template <int KB, int VB>
hipError_t launch_dt(const AppendArgs& a, int dtype, int d, hipStream_t s) {
  if (dtype == 0) return launch_d<KB, VB, 0>(a, d, s);
  if (dtype == 1) return launch_d<KB, VB, 1>(a, d, s);
  if (dtype == 2) return launch_d<KB, VB, 2>(a, d, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int kbits, int vbits, int dtype, int d, hipStream_t s) {
  if (kbits == 16 && vbits == 16) return launch_dt<16, 16>(a, dtype, d, s);
  if (kbits == 8 && vbits == 8) return launch_dt<8, 8>(a, dtype, d, s);
  if (kbits == 8 && vbits == 4) return launch_dt<8, 4>(a, dtype, d, s);
  if (kbits == 4 && vbits == 8) return launch_dt<4, 8>(a, dtype, d, s);
  if (kbits == 4 && vbits == 4) return launch_dt<4, 4>(a, dtype, d, s);
  if (kbits == kF8 && vbits == 4) return launch_dt<kF8, 4>(a, dtype, d, s);
  return hipErrorInvalidValue;
}

}  // namespace kvq

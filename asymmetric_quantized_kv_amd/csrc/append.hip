// Quantize-on-append: new tokens' keys and values are encoded block by block and
// written at the end of the session cache ("KVSplit -- contexto 2 a 3 vezes mais longo
// em Apple Silicon", section "Opinioes no Hacker News": the cache is quantized at run
// time as tokens are processed; bit widths per "Principais resultados de benchmark").
//
// One lane owns one 32-element block: it loads the block (64 or 128 bytes), takes its amax
// and scale once, and writes the block's codes (16 to 64 bytes) and scale; a wave covers
// 64 / (D / 32) consecutive tokens of one KV head, so its stores fill consecutive rows of the
// head's planes.  (Four lanes per block, each with 8 elements, redo the scale four times
// and exchange the amax: more VALU work, which bounds this kernel.)  Rounding follows the
// format fixed in include/kvq.h: fp32 IEEE division, fp16 round-to-nearest-even for the
// scale, round-half-away for the codes.  The per-element quotients come from a reciprocal
// and an fma correction that give the IEEE quotient's codes (see encode_one).
// fp8 keys (OCP MX blocks: a power-of-two block scale and E4M3 codes, the FP8
// alternative of "KV Cache Offloading for Context-Intensive Tasks", section
// "2. Metodologia") take the exponent from the amax's fp32 bits; the division by a
// power of two is exact and the E4M3 rounding is done in fp32 integer steps.
#include <algorithm>

#include "kvq_internal.h"

namespace kvq {
namespace {

// Eight elements of type DT (0 fp32, 1 bf16, 2 fp16) from their raw bytes (32 or 16) as fp32.
template <int DT>
__device__ __forceinline__ void unpack8(const uint4* raw, float* x) {   // x[0 .. 8)
  if constexpr (DT == 0) {  // fp32
    const uint4 a = raw[0], b = raw[1];
    x[0] = __uint_as_float(a.x); x[1] = __uint_as_float(a.y); x[2] = __uint_as_float(a.z); x[3] = __uint_as_float(a.w);
    x[4] = __uint_as_float(b.x); x[5] = __uint_as_float(b.y); x[6] = __uint_as_float(b.z); x[7] = __uint_as_float(b.w);
  } else {
    const uint4 v = raw[0];
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

// Code dwords of one 32-element block: 16 (fp16), 8 (8-bit and fp8) or 4 (4-bit).
template <int BITS>
constexpr int block_words() { return BITS == 16 ? 16 : (BITS == 4 ? 4 : 8); }

// Encode one 32-element block x of a row into its code dwords w; the scale goes to
// scales_row + (block offset).
template <int BITS>
__device__ __forceinline__ void encode_block(const float (&x)[kBlock], uint32_t (&w)[block_words<BITS>()],
                                             uint8_t* scales_row, int blk) {
  float amax = 0.f;
  if constexpr (BITS != 16) {
#pragma unroll
    for (int i = 0; i < kBlock; ++i) amax = fmaxf(amax, fabsf(x[i]));
  }
  if constexpr (BITS == 16) {
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = f16_bits(x[2 * i]) | ((uint32_t)f16_bits(x[2 * i + 1]) << 16);
  } else if constexpr (BITS == kF8) {
    // e = floor(log2 amax) - 8 (the exponent of E4M3's largest binade), in [-127, 127];
    // a zero or subnormal amax gives -127
    const int eb = (int)((__float_as_uint(amax) >> 23) & 255);
    const int e = eb == 0 ? -127 : max(eb - 127 - 8, -127);
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);       // 2^-e, normal
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = 0;
#pragma unroll
    for (int i = 0; i < kBlock; ++i) w[i / 4] |= e4m3_code(x[i] * inv) << (8 * (i & 3));
    scales_row[blk] = (uint8_t)(e + 127);
  } else {
    constexpr float qmax = BITS == 8 ? 127.f : 7.f;
    const float raw = amax / qmax;                        // IEEE division
    const float d32 = fminf(raw, 65504.f);                // saturate
    const _Float16 d16 = (_Float16)d32;                   // round to nearest even
    const float d = (float)d16;
    // y = x / d without a division per element: r = RN(1 / d) from the hardware reciprocal
    // (within 1 ulp) and one Newton step, which lands on RN(1 / d) for every positive fp16 d;
    // then one Markstein correction of the quotient x r.  The corrected quotient is within
    // 0.5 ulp + 3 * 2^-24 ulp of x / d, so its code (round half away) can differ from the
    // IEEE quotient's only next to a rounding boundary (k + 1/2) d, and there (every fp16 d,
    // k <= 127) it equals the quotient bit for bit: the codes are the division's.  A block
    // with d == 0 or an infinite element (rare) divides as before.
    float y[kBlock];
    if (d != 0.f && amax <= 3.40282347e38f) {
      float r = __builtin_amdgcn_rcpf(d);
      r = fmaf(fmaf(-d, r, 1.f), r, r);
#pragma unroll
      for (int i = 0; i < kBlock; ++i) {
        const float t = x[i] * r;
        y[i] = fmaf(fmaf(-d, t, x[i]), r, t);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kBlock; ++i) y[i] = d != 0.f ? x[i] / d : 0.f;   // IEEE division
    }
    // round half away from zero, then clamp: trunc(clamp(y + copysign(1/2 - 2^-25, y))).  The
    // addend just below 1/2 keeps |y| = 1/2 - 2^-25 from rounding up to 1 in the addition,
    // while a tie k + 1/2 still rounds up to k + 1 (every fp32 |y| in [2^-30, 512) checked
    // against round-half-away; below that both give 0, above it both clamp).
    // The clamp can only act when d is below fp16's normal range (its rounding there may lose
    // far more than 2^-11) or saturated: otherwise d >= (amax / qmax)(1 - 2^-11 - 2^-23), so
    // |y| <= qmax (1 + 2^-10) < qmax + 1/2 for every element of the block.  A wave none of
    // whose blocks has such a d skips it.
    const bool clamp = d < 6.103515625e-05f || raw > 65504.f;
    int q[kBlock];
    if (__builtin_amdgcn_ballot_w64(clamp) != 0) {
#pragma unroll
      for (int i = 0; i < kBlock; ++i) {
        const float t = y[i] + __builtin_copysignf(0.49999997f, y[i]);
        q[i] = (int)fminf(fmaxf(t, -qmax), qmax);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kBlock; ++i) q[i] = (int)(y[i] + __builtin_copysignf(0.49999997f, y[i]));
    }
    if constexpr (BITS == 8) {
      // low bytes of four codes into one dword: two byte permutes (0x0c selects a zero byte)
#pragma unroll
      for (int h = 0; h < 8; ++h)
        w[h] = __builtin_amdgcn_perm((uint32_t)q[4 * h + 1], (uint32_t)q[4 * h], 0x0c0c0400u) |
               __builtin_amdgcn_perm((uint32_t)q[4 * h + 3], (uint32_t)q[4 * h + 2], 0x04000c0cu);
    } else {
#pragma unroll
      for (int h = 0; h < 4; ++h) w[h] = 0;
#pragma unroll
      for (int i = 0; i < kBlock; ++i) w[i / 8] |= (uint32_t)(q[i] + 8) << (4 * (i & 7));
    }
    *reinterpret_cast<uint16_t*>(scales_row + blk * 2) = __builtin_bit_cast(uint16_t, d16);
  }
}

// Grid: x = KV head, y over (token, block) pairs of that head (D / 32 lanes per token, one
// block a lane), z = keys / values.  The head runs fastest in dispatch order, so the
// workgroups in flight read rows of every head at once (the rows of one head lie hkv * D
// elements apart; the workgroups of a single head alone would keep to a fraction of the
// memory channels).  All index arithmetic is 32-bit shifts and masks.  Every workgroup of a
// call fits the device at once: each loads, encodes and stores one block a lane.  (Lanes
// that walk several turns, the next turn's loads ahead of the current turn's stores, ran
// slower; so did loads and stores staged through LDS to make each instruction contiguous.)
template <int BITS, int DT, int D>
__device__ __forceinline__ void append_rows(const AppendArgs& a, const void* src, uint8_t* codes, uint8_t* scales,
                                            int code_row, int scale_row) {
  constexpr int LPT = D / kBlock;                     // lanes (blocks) per token
  constexpr int SH = LPT == 2 ? 1 : 2;
  static_assert((1 << SH) == LPT, "head_dim 64 or 128");
  constexpr int W = block_words<BITS>();
  const uint32_t t = blockIdx.y * 256u + threadIdx.x;
  const uint32_t tok = t >> SH;
  if (tok >= (uint32_t)a.n) return;
  const int blk = (int)(t & (LPT - 1));
  const int64_t elem = ((int64_t)tok * a.hkv + blockIdx.x) * D + blk * kBlock;
  float x[kBlock];
  if constexpr (DT == 0) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(src) + elem);
#pragma unroll
    for (int i = 0; i < kBlock; i += 8) unpack8<DT>(p + i / 4, x + i);
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + elem);
#pragma unroll
    for (int i = 0; i < kBlock; i += 8) unpack8<DT>(p + i / 8, x + i);
  }
  uint32_t w[W];
  encode_block<BITS>(x, w, scales + (a.t0 + tok) * scale_row, blk);
  uint4* dst = reinterpret_cast<uint4*>(codes + (a.t0 + tok) * code_row + 4 * W * blk);
#pragma unroll
  for (int i = 0; i < W; i += 4) dst[i / 4] = make_uint4(w[i], w[i + 1], w[i + 2], w[i + 3]);
}

template <int KB, int VB, int DT, int D>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  uint8_t* region = a.layer_base + (int64_t)blockIdx.x * a.g.region();
  if (blockIdx.z == 0)
    append_rows<KB, DT, D>(a, a.src[0], region + a.g.off_kc(), region + a.g.off_ks(), a.g.kc, a.g.ks);
  else
    append_rows<VB, DT, D>(a, a.src[1], region + a.g.off_vc(), region + a.g.off_vs(), a.g.vc, a.g.vs);
}

template <int KB, int VB, int DT, int D>
hipError_t launch_t(const AppendArgs& a, hipStream_t s) {
  if (a.hkv > 0x7fffffff) return hipErrorInvalidValue;
  // grid y holds at most 65535 workgroups of 256 / (D / 32) tokens: longer appends go in pieces
  constexpr int64_t kTokensPerLaunch = 65535LL * (256 / (D / kBlock));
  const int64_t esize = DT == 0 ? 4 : 2;
  for (int64_t t0 = 0; t0 < a.n; t0 += kTokensPerLaunch) {
    AppendArgs p = a;
    p.n = std::min<int64_t>(kTokensPerLaunch, a.n - t0);
    p.t0 = a.t0 + t0;
    for (int i = 0; i < 2; ++i) p.src[i] = static_cast<const uint8_t*>(a.src[i]) + t0 * a.hkv * D * esize;
    const int64_t blocks = (p.n * (D / kBlock) + 255) / 256;
    hipLaunchKernelGGL((append_kernel<KB, VB, DT, D>), dim3((unsigned)a.hkv, (unsigned)blocks, 2), dim3(256), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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

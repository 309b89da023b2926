// Chunked "only the new tokens" prefill: the last n_new cached positions attend,
// causally, to everything cached so far, their own chunk read back quantized
// ("Reutilizacao de Cache KV para Conversas Longas no Apple Silicon Oferece Aceleracao
// de 200x", section "Principais Descobertas e Benchmarks": keep the cache between turns
// and process only the new tokens).  Rows are (new token, query head of the group),
// token-major, so a tile of rows spans few positions and the causal edge stays narrow.
//
// Q.K^T and P.V are dense contractions and run on the matrix cores
// (v_mfma_f32_32x32x16_f16).  Operands are fp16 rather than bf16: a code times an fp16
// scale needs more than bf16's 8 significant bits (a 1-key attention would return the
// value with a 2^-9 relative error), while fp16 keeps 11 bits at the same MFMA rate.
// A quantized key (code * scale: up to 18 significant bits) is carried as its fp16 rounding
// hi plus the rest lo = code * scale - hi, which fp16 holds exactly.  hi meets the query on
// the fp16 MFMA.  lo, at most 2^-11 of the key, goes to LDS in fp6 (E2M3; head_dim 128 with
// 16-bit queries) or fp8 (E4M3) with a power-of-two scale per 32-element block, and meets a
// copy of the query in the same format (also block-scaled) on the block-scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4) at four (fp6) or two (fp8) times the fp16 rate: its
// rounding stays 2^-17 (fp6) or 2^-20 (fp8) below the block's largest key, against fp16's
// 2^-12 of every key.  fp32 queries are carried as fp16 hi + lo.
// fp8 (E4M3) keys with power-of-two block scales widen to fp16 exactly in one conversion
// (v_cvt_scalef32_pk_f16_fp8), so they need no low part: one MFMA per k-step.  With bf16
// queries they are not widened at all: Q.K^T runs in OCP MX fp8 on the block-scaled MFMA,
// the cache's codes and block exponents against an exact two-part E4M3 split of the query.
//
// A workgroup owns 256 rows of one KV head and one split of the context.
// Per 64-key tile: the workgroup dequantizes K into LDS as [key][d] and V as [d][key]
// (packed fp16 arithmetic on magic-number conversions of the codes), while the raw
// codes of the next tile are already in flight; each wave computes S^T = K Q^T (lane =
// query row, 16 keys per 32-key block), keeps an online softmax per row, and accumulates
// O^T += V^T P^T.  P is used in the key order the S^T accumulator already has, and V^T is
// stored in that same order (vt_slot), so no register shuffle sits between the two
// contractions and each V^T operand is one 16-byte LDS read.
// The running max only moves when a row's tile max exceeds it by more than 2^8
// (probabilities up to 256 stay exact in fp16), which makes the rescale of the
// accumulators rare; the tile max itself is only taken when the weights formed against the
// running max could exceed that headroom.
#include "kvq_internal.h"
#include "buffer_ops.h"
#include "wave_ops.h"

#include <type_traits>

namespace kvq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef int int8v_t __attribute__((ext_vector_type(8)));
typedef short short2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half32_t __attribute__((ext_vector_type(32)));
typedef unsigned int uint6v_t __attribute__((ext_vector_type(6)));

constexpr float kLazyMax = 8.f;   // log2 headroom before the running max is moved
constexpr float kLazyWeight = 256.f;   // 2^kLazyMax: the largest weight the headroom allows

__device__ __forceinline__ half2_t h2(uint32_t x) { return __builtin_bit_cast(half2_t, x); }
__device__ __forceinline__ uint32_t u32(half2_t x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ __forceinline__ half2_t hconst(float a) {
  half2_t r;
  r.x = (_Float16)a;
  r.y = (_Float16)a;
  return r;
}
__device__ __forceinline__ half2_t splat(uint16_t b) {
  const _Float16 h = __builtin_bit_cast(_Float16, b);
  half2_t r;
  r.x = h;
  r.y = h;
  return r;
}

// max and sum of lanes i and i ^ 32 (v_permlane32_swap: no LDS round trip)
__device__ __forceinline__ float swap32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Power-of-two prescale of a wave's query rows, lane_amax being the largest |q| among this
// lane's elements: returns 2^(127 - sb), which puts the wave's largest |q| in [2^14, 2^15),
// and sets *score_scale = qk_scale 2^(sb - 127).  Both are wave-uniform; the score scale is
// formed by adding to qk_scale's exponent field (integer work on scalar registers), so sb is
// clamped to keep that exponent normal (a query needs it only beyond 2^100 or below 2^-100),
// and a zero, subnormal or non-finite qk_scale takes no prescale.
__device__ __forceinline__ float wave_prescale(float lane_amax, float qk_scale, float* score_scale) {
  const uint32_t qb = __float_as_uint(qk_scale);
  const int eq = (int)((qb >> 23) & 255);
  int sb = max((int)((__float_as_uint(wave_max(lane_amax)) >> 23) & 255) - 14, 1);
  sb = eq == 0 || eq == 255 ? 127 : min(max(sb, 128 - eq), 381 - eq);
  *score_scale = __uint_as_float(qb + ((uint32_t)(sb - 127) << 23));
  return __uint_as_float((uint32_t)(254 - sb) << 23);
}

// The block-scaled product of the key low parts (format F: 0 = fp8 E4M3, 2 = fp6 E2M3, both
// operands) with the key scale taken from byte mm of ka (the instruction's byte select, which
// must be a constant) and the query scale from qa.
template <int F>
__device__ __forceinline__ float16_t scaled_mfma(int mm, const int8v_t& a, const int8v_t& b, const float16_t& c,
                                                 uint32_t ka, uint32_t qa) {
  return mm == 0 ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, F, F, 0, (int)ka, 0, (int)qa)
                 : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, F, F, 1, (int)ka, 0, (int)qa);
}

// four fp16 values / 2^t as four E4M3 bytes (the conversion divides by its scale operand)
__device__ __forceinline__ uint32_t fp8x4(half2_t a, half2_t b, float scale) {
  short2_t r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(r, a, scale, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(r, b, scale, true);
  return __builtin_bit_cast(uint32_t, r);
}

// Slot of key group g (keys 4 g .. 4 g + 3) in a transposed-value row: within each 16 keys the
// groups go in the order 0, 2, 1, 3, so that the keys a lane half takes for one P.V product
// (4 hl + 0..3 and 8 + 4 hl + 0..3 of the 16, the order of the S^T accumulator) are adjacent.
__device__ __forceinline__ int vt_slot(int g) { return (g & ~3) | ((g & 1) << 1) | ((g >> 1) & 1); }

// fp16 magic numbers: 0x64xx reads as 1024 + xx when xx < 4 bits of exponent room, so
// a code placed in the low mantissa bits comes back exactly after one packed subtract.
constexpr uint32_t kMagic = 0x64646464u;
constexpr uint32_t kHalfBias1024 = 0x64006400u;

// the 4 codes of one dword of 8-bit keys as fp16 pairs (e0, e1), (e2, e3)
__device__ __forceinline__ void k8_pairs(uint32_t w, half2_t (&c)[2]) {
  const uint32_t x = w ^ 0x80808080u;                                            // c + 128
  c[0] = h2(__builtin_amdgcn_perm(kMagic, x, 0x04010400u)) - hconst(1152.f);
  c[1] = h2(__builtin_amdgcn_perm(kMagic, x, 0x04030402u)) - hconst(1152.f);
}

// (x & mask) | bits in one v_and_or_b32 (its VOP3 form takes no literal operand, so the
// compiler would emit an and and an or); bits comes in a register
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t bits) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(bits));
  return r;
}

// the 8 codes of one dword of 4-bit keys as fp16 pairs (e2j, e2j+1), j = 0..3; bias holds
// kHalfBias1024
__device__ __forceinline__ void k4_pairs(uint32_t w, uint32_t bias, half2_t (&c)[4]) {
  const uint32_t w4 = w >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t sel = (uint32_t)j | ((uint32_t)(4 + j) << 16) | 0x0c000c00u;  // [w.bj, 0, w4.bj, 0]
    const uint32_t p = __builtin_amdgcn_perm(w4, w, sel);
    c[j] = h2(and_or(p, 0x000F000Fu, bias)) - hconst(1032.f);
  }
}

// The key low part's format: 3 = fp6 (E2M3), 2 = fp8 (E4M3), both with power-of-two block
// scales on the block-scaled MFMA; 0 = none (fp16 and fp8 keys are exact in fp16).  fp6 needs
// a whole block per producer thread (head_dim 128), and fp32 queries keep fp8 (the fp6 query
// exchange would spill their registers in the tile loop).
template <int KB, int D, bool QSPLIT>
constexpr int key_lo_format() {
  return KB == 16 || KB == kF8 ? 0 : (D == 128 && !QSPLIT ? 3 : 2);
}

// MX (fp8 keys with bf16 queries): Q.K^T on the block-scaled MFMA in OCP MX fp8.  The keys are
// the cache's own E4M3 codes and block exponents, copied to LDS as they are; each bf16 query
// is split into two E4M3 parts with power-of-two scales per 32-element block, hi (its top four
// significant bits) and lo (the rest, exact for bf16), so the products are those of the exact
// query.  Two MX products per 64 key elements take the issue time of the four fp16 ones.
template <int KB, int VB, int D, bool QSPLIT, bool MX = false>
__global__ __launch_bounds__(kChunkThreads) void chunk_kernel(ChunkArgs a) {
  static_assert(!MX || (KB == kF8 && !QSPLIT), "MX products: fp8 keys, 16-bit queries");
  constexpr int KLO = key_lo_format<KB, D, QSPLIT>();
  constexpr bool KSPLIT = KLO != 0;
  constexpr int NK = kChunkKeys;   // keys per tile
  constexpr int KSTR = D + 8;      // halves per LDS key row
  // halves per LDS transposed-value row: 36 dwords, so that the 16-byte reads of 8 lanes down a
  // column fall in distinct banks
  constexpr int VSTR = NK + 8;
  constexpr int NDT = D / 32;      // 32-wide output blocks along d
  constexpr int NKS = D / 16;      // k-steps of Q.K^T
  constexpr int KE = D / 4;        // key elements one producer thread dequantizes (4 per key)
  constexpr int KW = KE * (KB == kF8 ? 8 : KB) / 32;  // their dwords
  constexpr int VW = VB / 4;       // dwords of 8 value elements of one key
  constexpr int VITEMS = (NK / 4) * (D / 8);  // (4 keys x 8 d) value items per tile
  constexpr int KBUF = NK * KSTR, VBUF = D * VSTR;
  // fp8 / fp6 low parts: LDS rows of D bytes (+16: conflict-free 16-byte reads down a column;
  // an fp6 block takes 24 of its 32 bytes), and per key and block the E8M0 exponent of its
  // scale, ordered [h][m] for block 2 m + h (the scaled MFMA takes the scale of block 2 m + h
  // of its m-th product from lane half h)
  constexpr int NB = D / kBlock, NBH = NB / 2, LSTR = D + 16;
  constexpr int K8STR = D + 16;    // MX: bytes per LDS key row of E4M3 codes
  static_assert(kChunkThreads == 768 && kChunkRows == 256, "8 consumer + 4 producer waves");
  // two tile buffers: the producers fill one while the consumers read the other
  __shared__ __attribute__((aligned(16))) _Float16 s_k[MX ? NK * K8STR : 2 * KBUF];   // MX: codes, bytes
  __shared__ __attribute__((aligned(16))) uint8_t s_kl8[KLO >= 2 ? 2 * NK * LSTR : 16];
  __shared__ __attribute__((aligned(4))) uint8_t s_kls[KLO >= 2 || MX ? 2 * NK * NB : 4];
  __shared__ __attribute__((aligned(16))) uint8_t s_q8[KLO >= 2 ? kChunkRows * LSTR : 16];  // fp8 / fp6 queries
  __shared__ __attribute__((aligned(16))) _Float16 s_vt[2 * VBUF];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool producer = wave >= 8;
  // Workgroups are dealt round-robin to the 8 XCDs.  Renumber them so that the row
  // tiles of one (KV head, split), which all stream the same keys and values, sit on
  // one XCD and share its L2.
  int mt, head, split;
  {
    const uint32_t n_mt = gridDim.x, n = gridDim.x * gridDim.y * gridDim.z;
    const uint32_t lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const uint32_t xcd = lin % kXcds, per = n / kXcds, rem = n % kXcds;
    const uint32_t t = xcd * per + min(xcd, rem) + lin / kXcds;   // bijection on [0, n)
    mt = (int)(t % n_mt);
    head = (int)((t / n_mt) % gridDim.y);
    split = (int)(t / (n_mt * gridDim.y));
  }
  const int64_t rows = a.n_new * a.group;
  const int64_t tile_r0 = (int64_t)mt * kChunkRows;
  const int64_t base_pos = a.len - a.n_new;

  const int64_t region = a.g.region();
  const uint8_t* kc = a.base + (int64_t)head * region;
  const uint8_t* ks = kc + a.g.off_ks();
  const uint8_t* vc = kc + a.g.off_vc();
  const uint8_t* vs = kc + a.g.off_vs();

  const int64_t k_lo = (int64_t)split * a.tps;
  const int64_t k_hi = min(k_lo + a.tps, a.len);
  const int64_t last_row = min(tile_r0 + kChunkRows, rows) - 1;
  const int64_t k_end = min(k_hi, base_pos + last_row / a.group + 1);
  const int n_tiles = k_end > k_lo ? (int)((k_end - k_lo + NK - 1) / NK) : 0;
  // tiles before n_safe are visible to every row of the workgroup: no mask work
  const int64_t wg_min_pos = base_pos + tile_r0 / a.group;
  const int n_safe = (int)max((int64_t)0, (min(k_end, wg_min_pos + 1) - k_lo) / NK);

  if (producer) {
    // ================= producers: fetch codes, dequantize into the free buffer ==========
    const int pt = tid - 512;
    const int k_key = pt >> 2, k_part = pt & 3;
    const int v_kg = pt & 15, v_dg = pt >> 4;
    const bool v_on = pt < VITEMS;
    const uint32_t k_off = k_key * a.g.kc + k_part * (KW * 4);
    const uint32_t ks_off = k_key * a.g.ks + (KB == kF8 ? 1 : 2) * ((k_part * KE) / kBlock);
    const uint32_t v_off = 4 * v_kg * a.g.vc + v_dg * VB;
    const uint32_t vs_off = 4 * v_kg * a.g.vs + 2 * (v_dg >> 2);
    uint32_t kraw[KW];
    uint16_t kscale = 0;
    uint32_t vraw[4][VW];
    uint16_t vscale[4] = {0, 0, 0, 0};
    // the tile's rows of each plane through a buffer resource based at the tile (64-bit
    // tile offsets in scalar registers, per-thread 32-bit offsets fixed)
    auto fetch = [&](int t) {
      const int64_t kt0 = k_lo + (int64_t)t * NK;
      buf_dwords<KW>(make_rsrc(kc + kt0 * a.g.kc, NK * a.g.kc), k_off, 0, kraw);
      if constexpr (KB == kF8) kscale = buf_u8(make_rsrc(ks + kt0 * a.g.ks, NK * a.g.ks), ks_off, 0);
      else if constexpr (KB != 16) kscale = buf_u16(make_rsrc(ks + kt0 * a.g.ks, NK * a.g.ks), ks_off, 0);
      if (v_on) {
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vc + kt0 * a.g.vc, NK * a.g.vc);
        const __amdgpu_buffer_rsrc_t rvs = make_rsrc(vs + kt0 * a.g.vs, NK * a.g.vs);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          buf_dwords<VW>(rv, v_off, kk * a.g.vc, vraw[kk]);
          if constexpr (VB != 16) vscale[kk] = buf_u16(rvs, vs_off, kk * a.g.vs);
        }
      }
    };
    uint32_t bias;   // kHalfBias1024 in a register for and_or, set once
    asm volatile("v_mov_b32 %0, %1" : "=v"(bias) : "i"(kHalfBias1024));
    auto produce = [&](int buf) {
      _Float16* bk = s_k + buf * KBUF;
      _Float16* bv = s_vt + buf * VBUF;
      if constexpr (MX) {
        // the codes as they are (KE bytes at byte KE k_part of the key's row) and the block
        // exponent, ordered [h][m] for block 2 m + h like the low parts' scales
        uint8_t* b8 = reinterpret_cast<uint8_t*>(s_k) + buf * NK * K8STR + k_key * K8STR + k_part * KE;
#pragma unroll
        for (int i = 0; i < KW / 4; ++i)
          *reinterpret_cast<uint4*>(b8 + 16 * i) = make_uint4(kraw[4 * i], kraw[4 * i + 1], kraw[4 * i + 2], kraw[4 * i + 3]);
        if constexpr (KW % 4 != 0) static_assert(KW % 4 == 0, "16-byte code runs");
        const int b = (k_part * KE) / kBlock;
        if ((k_part * KE) % kBlock == 0) s_kls[buf * NK * NB + k_key * NB + (b & 1) * NBH + (b >> 1)] = (uint8_t)kscale;
      } else {
        half2_t hi[KE / 2], lo[KE / 2];
        if constexpr (KB == 16) {
#pragma unroll
          for (int i = 0; i < KE / 2; ++i) hi[i] = h2(kraw[i]);
        } else if constexpr (KB == kF8) {
          // E4M3 value * 2^(s - 127), rounded once to fp16: exact while |x| < 65536
          // (s = 0 reads as 0: 2^-127 times any code is below every fp16)
          const float x = __uint_as_float((uint32_t)kscale << 23);
#pragma unroll
          for (int w = 0; w < KW; ++w) {
            hi[2 * w] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)kraw[w], x, false);
            hi[2 * w + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)kraw[w], x, true);
          }
        } else {
          const half2_t d2 = splat(kscale);
#pragma unroll
          for (int w = 0; w < KW; ++w) {
            if constexpr (KB == 8) {
              half2_t c[2];
              k8_pairs(kraw[w], c);
#pragma unroll
              for (int j = 0; j < 2; ++j) {
                hi[2 * w + j] = c[j] * d2;
                if constexpr (KSPLIT) lo[2 * w + j] = __builtin_elementwise_fma(c[j], d2, -hi[2 * w + j]);
              }
            } else {
              half2_t c[4];
              k4_pairs(kraw[w], bias, c);
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                hi[4 * w + j] = c[j] * d2;
                if constexpr (KSPLIT) lo[4 * w + j] = __builtin_elementwise_fma(c[j], d2, -hi[4 * w + j]);
              }
            }
          }
        }
#pragma unroll
        for (int i = 0; i < KE / 8; ++i) {
          const int off = k_key * KSTR + k_part * KE + 8 * i;
          *reinterpret_cast<uint4*>(&bk[off]) =
              make_uint4(u32(hi[4 * i]), u32(hi[4 * i + 1]), u32(hi[4 * i + 2]), u32(hi[4 * i + 3]));
        }
        if constexpr (KLO == 2) {
          // lo / 2^t as E4M3 with t = max(e, 1) - 26 for the fp16 exponent field e of the scale:
          // |code * scale| < 2^(e - 7) bounds |lo| by 2^(e - 19), so |lo| / 2^t <= 128 (and a
          // subnormal product's lo, below 2^-25, stays below 1)
          const int e = max((int)((kscale >> 10) & 31), 1);
          const float sc = __uint_as_float((uint32_t)(e + 101) << 23);
          uint8_t* bl = s_kl8 + buf * NK * LSTR + k_key * LSTR + k_part * KE;
#pragma unroll
          for (int i = 0; i < KE / 16; ++i)
            *reinterpret_cast<uint4*>(bl + 16 * i) =
                make_uint4(fp8x4(lo[8 * i], lo[8 * i + 1], sc), fp8x4(lo[8 * i + 2], lo[8 * i + 3], sc),
                           fp8x4(lo[8 * i + 4], lo[8 * i + 5], sc), fp8x4(lo[8 * i + 6], lo[8 * i + 7], sc));
          const int b = (k_part * KE) / kBlock;
          if ((k_part * KE) % kBlock == 0)
            s_kls[buf * NK * NB + k_key * NB + (b & 1) * NBH + (b >> 1)] = (uint8_t)(e + 101);
        } else if constexpr (KLO == 3) {
          // the thread's block (KE = 32) as E2M3 / 2^t, t = max(e, 1) + bits - 29: with
          // |code| <= 2^(bits - 1), |lo| <= 2^(e + bits - 27), so |lo| / 2^t <= 4 (E2M3 tops out
          // at 7.5 and saturates); 24 bytes at byte 32 b of the key's row
          const int e = max((int)((kscale >> 10) & 31), 1);
          const int t = e + KB - 29;
          const float sc = __uint_as_float((uint32_t)(t + 127) << 23);
          half32_t lv;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            lv[2 * i] = lo[i].x;
            lv[2 * i + 1] = lo[i].y;
          }
          const uint6v_t f = __builtin_amdgcn_cvt_scalef32_pk32_fp6_f16(lv, sc);
          uint8_t* bl = s_kl8 + buf * NK * LSTR + k_key * LSTR + k_part * kBlock;
          *reinterpret_cast<uint4*>(bl) = make_uint4(f[0], f[1], f[2], f[3]);
          *reinterpret_cast<uint2*>(bl + 16) = make_uint2(f[4], f[5]);
          s_kls[buf * NK * NB + k_key * NB + (k_part & 1) * NBH + (k_part >> 1)] = (uint8_t)(t + 127);
        }
      }
      if (v_on) {
        // keys (0, 1) and (2, 3) side by side per element: pr[e][pair] = (v_2p, v_2p+1)
        uint32_t pr[8][2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const uint32_t* wa = vraw[2 * p];
          const uint32_t* wb = vraw[2 * p + 1];
          half2_t d2 = hconst(1.f);
          if constexpr (VB != 16) {
            d2.x = __builtin_bit_cast(_Float16, vscale[2 * p]);
            d2.y = __builtin_bit_cast(_Float16, vscale[2 * p + 1]);
          }
          if constexpr (VB == 4) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint32_t sel = (uint32_t)j | ((uint32_t)(4 + j) << 16) | 0x0c000c00u;  // [a.bj, 0, b.bj, 0]
              const uint32_t q = __builtin_amdgcn_perm(wb[0], wa[0], sel);
              const half2_t ce = h2(and_or(q, 0x000F000Fu, bias)) - hconst(1032.f);
              // high nibbles: 1024 + 16 u, so u - 8 = x / 16 - 72 (exact)
              const half2_t co = __builtin_elementwise_fma(h2(and_or(q, 0x00F000F0u, bias)), hconst(0.0625f),
                                                           hconst(-72.f));
              pr[2 * j][p] = u32(ce * d2);
              pr[2 * j + 1][p] = u32(co * d2);
            }
          } else if constexpr (VB == 8) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              const uint32_t xa = wa[i] ^ 0x80808080u, xb = wb[i] ^ 0x80808080u;
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const uint32_t sel = (uint32_t)j | ((uint32_t)(4 + j) << 16) | 0x0c000c00u;
                const uint32_t q = __builtin_amdgcn_perm(xb, xa, sel) | kHalfBias1024;
                pr[4 * i + j][p] = u32((h2(q) - hconst(1152.f)) * d2);
              }
            }
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              pr[2 * i][p] = __builtin_amdgcn_perm(wb[i], wa[i], 0x05040100u);
              pr[2 * i + 1][p] = __builtin_amdgcn_perm(wb[i], wa[i], 0x07060302u);
            }
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
          *reinterpret_cast<uint2*>(&bv[(8 * v_dg + e) * VSTR + 4 * vt_slot(v_kg)]) = make_uint2(pr[e][0], pr[e][1]);
      }
    };
    if (n_tiles > 0) {
      fetch(0);
      produce(0);
      if (n_tiles > 1) fetch(1);
    }
    __syncthreads();
    for (int t = 0; t < n_tiles; ++t) {
      if (t + 1 < n_tiles) {
        produce((t + 1) & 1);                 // tile t + 1 into the buffer not being read
        if (t + 2 < n_tiles) fetch(t + 2);    // its successor's codes fly meanwhile
      }
      __syncthreads();
    }
    return;
  }

  // ================= consumers: 32 query rows per wave =================================
  const int hl = lane >> 5, col = lane & 31;
  const int64_t r0 = tile_r0 + wave * 32;
  const int64_t my_row = r0 + col;
  const bool valid = my_row < rows;
  const int64_t tok = valid ? my_row / a.group : 0;
  const int qh = head * a.group + (valid ? (int)(my_row % a.group) : 0);
  const int64_t pos = valid ? base_pos + tok : -1;
  const bool wave_active = r0 < rows;

  // Q^T as the B operand: lane (col, hl) holds d = 16 k + 8 hl .. + 7 of its row.  The wave's
  // rows are first scaled by a power of two 2^-k that puts their largest |q| in [2^14, 2^15),
  // so fp16 holds them for any magnitude (16-bit queries exactly); 2^k goes into the score
  // scale, one for the wave.
  half8_t qv[MX ? 1 : NKS];
  half8_t ql[QSPLIT ? NKS : 1];
  // MX: the B operands of the m-th product, E4M3 hi and lo parts of elements 64 m + 16 hl + 0..15
  // (bytes 0..15) and 64 m + 32 + 16 hl + 0..15 (bytes 16..31), and the exponents of block 2 m + hl
  int8v_t qhi[MX ? NBH : 1], qlo[MX ? NBH : 1];
  uint32_t qeh[MX ? NBH : 1], qel[MX ? NBH : 1];
  float qks;   // raw score -> base-2 logit (wave-uniform)
  if constexpr (MX) {
    // block b's 16 elements 32 b + 16 hl + 0..15 of this lane's row (its partner holds the other
    // 16): two 16-byte loads per block, all issued before the first conversion
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + (tok * a.hq + qh) * (int64_t)D +
                                                      16 * hl);
    uint4 raw[2 * NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      raw[2 * b] = valid ? src[4 * b] : make_uint4(0u, 0u, 0u, 0u);
      raw[2 * b + 1] = valid ? src[4 * b + 1] : make_uint4(0u, 0u, 0u, 0u);
    }
    qks = a.qk_scale;   // the products are those of the queries themselves
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint4 r = raw[2 * b + i / 8];
        const uint32_t w = (i & 7) < 2 ? r.x : (i & 7) < 4 ? r.y : (i & 7) < 6 ? r.z : r.w;
        x[i] = __uint_as_float((w >> (16 * (i & 1))) << 16);
      }
      float am = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(x[i]));
      am = swap32_max(am);
      // hi: x / 2^t in E4M3 with t = floor(log2 amax) - 7 (|x| / 2^t < 256, E4M3 holds up to 448);
      // lo = x - hi, a multiple of x's bf16 unit below half hi's, at 2^(t - 4): |lo| / 2^(t - 4)
      // <= 128 and four significant bits hold it (exact but where x is under 2^-13 of the amax).
      // Both exponents stay at or above -126, so each conversion scale is a normal float (a
      // zero block, or one under 2^-115, would otherwise give the remainder a scale of 0)
      const int t = max((int)((__float_as_uint(am) >> 23) & 255) - 134, -126);
      const int tl = max(t - 4, -126);
      const float sh = __uint_as_float((uint32_t)(t + 127) << 23), sl = __uint_as_float((uint32_t)(tl + 127) << 23);
      uint32_t h4[4], l4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        short2_t ph = {0, 0}, pl = {0, 0};
        ph = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(ph, x[4 * j], x[4 * j + 1], sh, false);
        ph = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(ph, x[4 * j + 2], x[4 * j + 3], sh, true);
        const uint32_t hw = __builtin_bit_cast(uint32_t, ph);
        const auto v01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)hw, sh, false);
        const auto v23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)hw, sh, true);
        pl = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(pl, x[4 * j] - v01[0], x[4 * j + 1] - v01[1], sl, false);
        pl = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(pl, x[4 * j + 2] - v23[0], x[4 * j + 3] - v23[1], sl, true);
        h4[j] = hw;
        l4[j] = __builtin_bit_cast(uint32_t, pl);
      }
      const int m = b >> 1, g = b & 1;   // bytes 16 g .. of the m-th product
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qhi[m][4 * g + j] = (int)h4[j];
        qlo[m][4 * g + j] = (int)l4[j];
      }
      if (g == hl) {
        qeh[m] = (uint32_t)(t + 127);
        qel[m] = (uint32_t)(tl + 127);
      }
    }
  } else {
    // 8 consecutive elements per k-step: one 16-byte load each (two for fp32), all issued
    // before the first conversion
    const int64_t qoff = (tok * a.hq + qh) * (int64_t)D + 8 * hl;
    if constexpr (QSPLIT) {   // fp32 queries
      const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(a.q) + qoff);
      float4 raw[2 * NKS];
#pragma unroll
      for (int k = 0; k < NKS; ++k) {
        raw[2 * k] = valid ? src[4 * k] : make_float4(0.f, 0.f, 0.f, 0.f);
        raw[2 * k + 1] = valid ? src[4 * k + 1] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      float am = 0.f;
#pragma unroll
      for (int k = 0; k < 2 * NKS; ++k)
        am = fmaxf(am, fmaxf(fmaxf(fabsf(raw[k].x), fabsf(raw[k].y)), fmaxf(fabsf(raw[k].z), fabsf(raw[k].w))));
      const float qi = wave_prescale(am, a.qk_scale, &qks);
#pragma unroll
      for (int k = 0; k < NKS; ++k) {
        const float x[8] = {raw[2 * k].x, raw[2 * k].y, raw[2 * k].z, raw[2 * k].w,
                            raw[2 * k + 1].x, raw[2 * k + 1].y, raw[2 * k + 1].z, raw[2 * k + 1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float y = x[i] * qi;
          qv[k][i] = (_Float16)y;
          ql[k][i] = (_Float16)(y - (float)qv[k][i]);
        }
      }
    } else {                  // bf16 or fp16 queries
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + qoff);
      uint4 raw[NKS];
#pragma unroll
      for (int k = 0; k < NKS; ++k) raw[k] = valid ? src[2 * k] : make_uint4(0u, 0u, 0u, 0u);
      const bool bf = a.q_dtype == 1;
      // the largest magnitude from the bits: without the sign, bf16 and fp16 magnitudes
      // order as their bit patterns
      uint32_t mb = 0;
#pragma unroll
      for (int k = 0; k < NKS; ++k) {
        const uint32_t w[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) mb = max(mb, max(w[j] & 0x7fffu, (w[j] >> 16) & 0x7fffu));
      }
      const float qi = wave_prescale(bf ? __uint_as_float(mb << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)mb),
                                     a.qk_scale, &qks);
#pragma unroll
      for (int k = 0; k < NKS; ++k) {
        const uint32_t w[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint16_t b = (uint16_t)(w[i / 2] >> (16 * (i & 1)));
          qv[k][i] = (_Float16)((bf ? __uint_as_float((uint32_t)b << 16) : (float)__builtin_bit_cast(_Float16, b)) * qi);
        }
      }
    }
  }

  // fp8 copy of this wave's query rows for the low parts of the keys: one power-of-two scale
  // 2^t per (row, block), t = floor(log2 amax) - 7 so that |q| / 2^t < 256 (2^-126 for a zero
  // block); qs8[m] holds the E8M0 exponent of block 2 m + hl, which this lane feeds the
  // scaled MFMA
  uint32_t qs8[KLO >= 2 ? NBH : 1];
  if constexpr (KLO == 2) {
    uint8_t* q8 = s_q8 + (wave * 32 + col) * LSTR;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float am = 0.f;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf((float)qv[2 * b + kk][i]));
      am = swap32_max(am);
      const int t = max((int)((__float_as_uint(am) >> 23) & 255) - 134, -126);
      const float sc = __uint_as_float((uint32_t)(t + 127) << 23);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const half8_t x = qv[2 * b + kk];
        const half2_t p0 = {x[0], x[1]}, p1 = {x[2], x[3]}, p2 = {x[4], x[5]}, p3 = {x[6], x[7]};
        *reinterpret_cast<uint2*>(q8 + 16 * (2 * b + kk) + 8 * hl) = make_uint2(fp8x4(p0, p1, sc), fp8x4(p2, p3, sc));
      }
      if ((b & 1) == hl) qs8[b >> 1] = (uint32_t)(t + 127);
    }
  } else if constexpr (KLO == 3) {
    // the fp6 product takes a whole block from each lane: lane half hl converts block 2 m + hl,
    // half of which its partner (lane ^ 32) holds; scale 2^t, t = floor(log2 amax) - 1, so
    // |q| / 2^t < 4 (E2M3 tops out at 7.5); 24 bytes at byte 32 (2 m + hl) of the row
    uint8_t* q6 = s_q8 + (wave * 32 + col) * LSTR;
#pragma unroll
    for (int mm = 0; mm < NBH; ++mm) {
      // elements 8 hl + i (run 0) and 16 + 8 hl + i (run 1) of blocks 2 mm and 2 mm + 1 are here;
      // send the partner those of the block it converts, receive those of ours
      // (selects, not an index by hl: a lane-dependent index would put qv in scratch memory)
      const half8_t mine0 = hl ? qv[4 * mm + 2] : qv[4 * mm], mine1 = hl ? qv[4 * mm + 3] : qv[4 * mm + 1];
      const half8_t send0 = hl ? qv[4 * mm] : qv[4 * mm + 2], send1 = hl ? qv[4 * mm + 1] : qv[4 * mm + 3];
      half8_t got0, got1;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x0 = __builtin_bit_cast(uint32_t, half2_t{send0[2 * w], send0[2 * w + 1]});
        const uint32_t x1 = __builtin_bit_cast(uint32_t, half2_t{send1[2 * w], send1[2 * w + 1]});
        const auto r0 = __builtin_amdgcn_permlane32_swap(x0, x0, false, false);
        const auto r1 = __builtin_amdgcn_permlane32_swap(x1, x1, false, false);
        const half2_t g0 = __builtin_bit_cast(half2_t, hl ? r0[0] : r0[1]);
        const half2_t g1 = __builtin_bit_cast(half2_t, hl ? r1[0] : r1[1]);
        got0[2 * w] = g0.x; got0[2 * w + 1] = g0.y;
        got1[2 * w] = g1.x; got1[2 * w + 1] = g1.y;
      }
      // the block in element order: 8-element runs r = 0..3 hold elements 8 r .. 8 r + 7
      half32_t blk;
      float am = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const _Float16 r0 = hl ? got0[i] : mine0[i];    // elements 0..7
        const _Float16 r1 = hl ? mine0[i] : got0[i];    // 8..15
        const _Float16 r2 = hl ? got1[i] : mine1[i];    // 16..23
        const _Float16 r3 = hl ? mine1[i] : got1[i];    // 24..31
        blk[i] = r0; blk[8 + i] = r1; blk[16 + i] = r2; blk[24 + i] = r3;
        am = fmaxf(am, fmaxf(fmaxf(fabsf((float)r0), fabsf((float)r1)), fmaxf(fabsf((float)r2), fabsf((float)r3))));
      }
      const int t = max((int)((__float_as_uint(am) >> 23) & 255) - 128, -126);
      const uint6v_t f = __builtin_amdgcn_cvt_scalef32_pk32_fp6_f16(blk, __uint_as_float((uint32_t)(t + 127) << 23));
      uint8_t* dst = q6 + 32 * (2 * mm + hl);
      *reinterpret_cast<uint4*>(dst) = make_uint4(f[0], f[1], f[2], f[3]);
      *reinterpret_cast<uint2*>(dst + 16) = make_uint2(f[4], f[5]);
      qs8[mm] = (uint32_t)(t + 127);
    }
  }

  float m = -INFINITY, l = 0.f;
  float mu = 0.f;   // the running max as the weights' offset (0 while the row has none)
  float16_t o[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[t][v] = 0.f;

  // one 32-key half of a tile: S^T = K Q^T, online softmax, O^T += V^T P^T
  auto half = [&](auto masked, const _Float16* bk, const uint8_t* bkl8, const uint8_t* bks, const _Float16* bv,
                  int64_t kt0, int st) __attribute__((always_inline)) {
    float16_t sv;
#pragma unroll
    for (int v = 0; v < 16; ++v) sv[v] = 0.f;
    if constexpr (MX) {
      // m-th pair of products: lane half hl brings bytes 16 hl .. + 15 of blocks 2 m and 2 m + 1
      // of its key's codes and the exponent of block 2 m + hl, against the query's hi and lo parts
      const uint8_t* kr = reinterpret_cast<const uint8_t*>(bk) + (32 * st + col) * K8STR + 16 * hl;
      const uint8_t* ksp = bks + (32 * st + col) * NB + hl * NBH;
      const uint32_t asc = NBH == 2 ? (uint32_t)*reinterpret_cast<const uint16_t*>(ksp) : (uint32_t)*ksp;
#pragma unroll
      for (int mm = 0; mm < NBH; ++mm) {
        const uint4 a0 = *reinterpret_cast<const uint4*>(kr + 64 * mm);
        const uint4 a1 = *reinterpret_cast<const uint4*>(kr + 64 * mm + 32);
        const int8v_t av8 = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        sv = scaled_mfma<0>(mm, av8, qhi[mm], sv, asc, qeh[mm]);
        sv = scaled_mfma<0>(mm, av8, qlo[mm], sv, asc, qel[mm]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < NKS; ++k) {
        const int off = (32 * st + col) * KSTR + 16 * k + 8 * hl;
        const half8_t ak = *reinterpret_cast<const half8_t*>(&bk[off]);
        sv = __builtin_amdgcn_mfma_f32_32x32x16_f16(ak, qv[k], sv, 0, 0, 0);
        if constexpr (QSPLIT) sv = __builtin_amdgcn_mfma_f32_32x32x16_f16(ak, ql[k], sv, 0, 0, 0);
      }
    }
    if constexpr (KLO == 2) {
      // m-th product: lane half hl brings bytes 16 hl .. + 15 of blocks 2 m and 2 m + 1, and the
      // scale of block 2 m + hl (16-byte group g of both halves is block 2 m + g)
      const uint8_t* kl = bkl8 + (32 * st + col) * LSTR + 16 * hl;
      const uint8_t* ql8 = s_q8 + (wave * 32 + col) * LSTR + 16 * hl;
      const uint8_t* ksp = bks + (32 * st + col) * NB + hl * NBH;
      const uint32_t asc = NBH == 2 ? (uint32_t)*reinterpret_cast<const uint16_t*>(ksp) : (uint32_t)*ksp;
#pragma unroll
      for (int mm = 0; mm < NBH; ++mm) {
        const uint4 a0 = *reinterpret_cast<const uint4*>(kl + 64 * mm);
        const uint4 a1 = *reinterpret_cast<const uint4*>(kl + 64 * mm + 32);
        const uint4 b0 = *reinterpret_cast<const uint4*>(ql8 + 64 * mm);
        const uint4 b1 = *reinterpret_cast<const uint4*>(ql8 + 64 * mm + 32);
        const int8v_t av8 = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        const int8v_t bv8 = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
        sv = scaled_mfma<0>(mm, av8, bv8, sv, asc, qs8[mm]);
      }
    } else if constexpr (KLO == 3) {
      // m-th product at the fp6 rate: lane half hl brings all 32 elements of block 2 m + hl (24
      // bytes) and that block's scale
      const uint8_t* kl = bkl8 + (32 * st + col) * LSTR + 32 * hl;
      const uint8_t* ql6 = s_q8 + (wave * 32 + col) * LSTR + 32 * hl;
      const uint8_t* ksp = bks + (32 * st + col) * NB + hl * NBH;
      const uint32_t asc = (uint32_t)*reinterpret_cast<const uint16_t*>(ksp);
#pragma unroll
      for (int mm = 0; mm < NBH; ++mm) {
        const uint4 a0 = *reinterpret_cast<const uint4*>(kl + 64 * mm);
        const uint2 a1 = *reinterpret_cast<const uint2*>(kl + 64 * mm + 16);
        const uint4 b0 = *reinterpret_cast<const uint4*>(ql6 + 64 * mm);
        const uint2 b1 = *reinterpret_cast<const uint2*>(ql6 + 64 * mm + 16);
        const int8v_t av6 = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, 0, 0};
        const int8v_t bv6 = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, 0, 0};
        sv = scaled_mfma<2>(mm, av6, bv6, sv, asc, qs8[mm]);
      }
    }
    if constexpr (decltype(masked)::value) {
      // keys kt0 + 32 st + [0, 32): offsets >= lim are past the range or in the future
      const int64_t kb0 = kt0 + 32 * st;
      const int lim = (int)max((int64_t)-1, min(min(k_end, pos + 1) - kb0, (int64_t)32));
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (8 * (v >> 2) + 4 * hl + (v & 3) >= lim) sv[v] = -INFINITY;
    }
    // online softmax, one query row per lane pair (col, col + 32).  The weights are formed
    // against the running max first: each is at most their sum, so a lane whose 16 weights
    // sum to at most 2^kLazyMax has no score past the max's headroom and needs no tile max.
    // Only when some lane's sum is larger (or its row has no max yet) is the tile max taken;
    // if it moves the running max, the accumulators are rescaled and the weights formed again.
    half8_t pb[2];
    auto weights = [&](float mu) __attribute__((always_inline)) {
      float s = 0.f;
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        half2_t pp;
        pp.x = (_Float16)__builtin_amdgcn_exp2f(fmaf(sv[v], qks, -mu));
        pp.y = (_Float16)__builtin_amdgcn_exp2f(fmaf(sv[v + 1], qks, -mu));
        s = __builtin_amdgcn_fdot2(pp, hconst(1.f), s, false);   // sum of the rounded weights
        pb[v >> 3][v & 7] = pp.x;
        pb[v >> 3][(v & 7) + 1] = pp.y;
      }
      return s;
    };
    float ls = weights(mu);
    if (__any(!(ls <= kLazyWeight) || m == -INFINITY)) {
      float mx = sv[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sv[v]);
      mx = swap32_max(mx) * qks;
      const bool move = mx > m + kLazyMax;
      if (__any(move)) {
        const float mn = move ? mx : m;
        const float alpha = __builtin_amdgcn_exp2f(m - (mn == -INFINITY ? 0.f : mn));
        l *= alpha;
#pragma unroll
        for (int t = 0; t < NDT; ++t)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[t][v] *= alpha;
        m = mn;
        mu = m == -INFINITY ? 0.f : m;
        ls = weights(mu);
      }
    }
    l += ls;
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        // keys 32 st + 16 kk + 4 hl + (0..3, 8..11), stored side by side (vt_slot): one 16-byte read
        const half8_t av = *reinterpret_cast<const half8_t*>(&bv[(32 * t + col) * VSTR + 32 * st + 16 * kk + 8 * hl]);
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, pb[kk], o[t], 0, 0, 0);
      }
    }
  };
  auto consume = [&](auto masked, int t) __attribute__((always_inline)) {
    if (wave_active) {
      const int buf = t & 1;
      const _Float16* bk = MX ? reinterpret_cast<const _Float16*>(reinterpret_cast<const uint8_t*>(s_k) + buf * NK * K8STR)
                              : s_k + buf * KBUF;
      const uint8_t* bkl8 = s_kl8 + (KLO >= 2 ? buf * NK * LSTR : 0);
      const uint8_t* bks = s_kls + (KLO >= 2 || MX ? buf * NK * NB : 0);
      const _Float16* bv = s_vt + buf * VBUF;
      const int64_t kt0 = k_lo + (int64_t)t * NK;
      half(masked, bk, bkl8, bks, bv, kt0, 0);
      half(masked, bk, bkl8, bks, bv, kt0, 1);
    }
    __syncthreads();
  };
  __syncthreads();   // tile 0 is in place
  int t = 0;
  for (; t < n_safe && t < n_tiles; ++t) consume(std::false_type{}, t);
  for (; t < n_tiles; ++t) consume(std::true_type{}, t);

  // ---- output -----------------------------------------------------------------------
  const float lt = swap32_sum(l);
  if (!valid) return;
  const int64_t orow = tok * a.hq + qh;
  if (!a.partial) {
    const float inv = 1.f / lt;
#pragma unroll
    for (int t2 = 0; t2 < NDT; ++t2)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * t2 + 8 * g4 + 4 * hl;
        float4 v = make_float4(o[t2][4 * g4] * inv, o[t2][4 * g4 + 1] * inv, o[t2][4 * g4 + 2] * inv,
                               o[t2][4 * g4 + 3] * inv);
        *reinterpret_cast<float4*>(a.out + orow * D + d) = v;
      }
  } else {
    float* p = a.ws + (orow * a.n_splits + split) * (D + 2);
#pragma unroll
    for (int t2 = 0; t2 < NDT; ++t2)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * t2 + 8 * g4 + 4 * hl;
#pragma unroll
        for (int i = 0; i < 4; ++i) p[d + i] = o[t2][4 * g4 + i];
      }
    if (hl == 0) {
      p[D] = m;
      p[D + 1] = lt;
    }
  }
}

template <int KB, int VB, int D, bool QSPLIT, bool MX = false>
const void* kernel_ptr() {
  return reinterpret_cast<const void*>(&chunk_kernel<KB, VB, D, QSPLIT, MX>);
}

template <int KB, int VB, int D>
hipError_t launch_t(const ChunkArgs& a, hipStream_t s) {
  const int64_t rows = a.n_new * a.group;
  const int64_t mt = (rows + kChunkRows - 1) / kChunkRows;
  dim3 grid((unsigned)mt, a.hkv, a.n_splits);
  if (a.q_dtype == 0)
    hipLaunchKernelGGL((chunk_kernel<KB, VB, D, true>), grid, dim3(kChunkThreads), 0, s, a);
  else if (KB == kF8 && a.q_dtype == 1)
    hipLaunchKernelGGL((chunk_kernel<KB, VB, D, false, KB == kF8>), grid, dim3(kChunkThreads), 0, s, a);
  else
    hipLaunchKernelGGL((chunk_kernel<KB, VB, D, false>), grid, dim3(kChunkThreads), 0, s, a);
  return hipGetLastError();
}

template <int KB, int VB>
hipError_t launch_d(const ChunkArgs& a, int d, hipStream_t s) {
  if (d == 64) return launch_t<KB, VB, 64>(a, s);
  if (d == 128) return launch_t<KB, VB, 128>(a, s);
  return hipErrorInvalidValue;
}

template <int KB, int VB>
const void* ptr_d(int d, bool q_fp32) {
  if (d == 64) return q_fp32 ? kernel_ptr<KB, VB, 64, true>() : kernel_ptr<KB, VB, 64, false>();
  return q_fp32 ? kernel_ptr<KB, VB, 128, true>() : kernel_ptr<KB, VB, 128, false>();
}

}  // namespace

hipError_t launch_chunk(const ChunkArgs& a, int kbits, int vbits, int d, hipStream_t s) {
  if (kbits == 16 && vbits == 16) return launch_d<16, 16>(a, d, s);
  if (kbits == 8 && vbits == 8) return launch_d<8, 8>(a, d, s);
  if (kbits == 8 && vbits == 4) return launch_d<8, 4>(a, d, s);
  if (kbits == 4 && vbits == 8) return launch_d<4, 8>(a, d, s);
  if (kbits == 4 && vbits == 4) return launch_d<4, 4>(a, d, s);
  if (kbits == kF8 && vbits == 4) return launch_d<kF8, 4>(a, d, s);
  return hipErrorInvalidValue;
}

// (The MX instantiation that fp8 keys take with bf16 queries holds, like this one, one
// workgroup per compute unit.)
const void* chunk_kernel_for(int kbits, int vbits, int d, bool q_fp32) {
  if (kbits == 16) return ptr_d<16, 16>(d, q_fp32);
  if (kbits == kF8) return ptr_d<kF8, 4>(d, q_fp32);
  if (kbits == 8 && vbits == 8) return ptr_d<8, 8>(d, q_fp32);
  if (kbits == 8) return ptr_d<8, 4>(d, q_fp32);
  if (vbits == 8) return ptr_d<4, 8>(d, q_fp32);
  return ptr_d<4, 4>(d, q_fp32);
}

}  // namespace kvq

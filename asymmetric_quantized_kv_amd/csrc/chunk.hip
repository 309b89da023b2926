// Chunked "only the new tokens" prefill: the last n_new cached positions attend,
// causally, to everything cached so far, their own chunk read back quantized
// ("Reutilizacao de Cache KV para Conversas Longas no Apple Silicon Oferece Aceleracao
// de 200x", section "Principais Descobertas e Benchmarks": keep the cache between turns
// and process only the new tokens).  Rows are (new token, query head of the group),
// token-major, so a tile of rows spans few positions and the causal edge stays narrow.
//
// Q.K^T and P.V are dense contractions and run on the matrix cores
// (v_mfma_f32_32x32x16_f16).  Operands are fp16 rather than bf16: codes times an fp16
// scale need more than bf16's 8 significant bits (a 1-key attention would return the
// value with a 2^-9 relative error), while fp16 keeps 11 bits at the same MFMA rate.
//
// A workgroup (4 waves) owns 128 rows of one KV head and one split of the context.
// Per 64-key tile: the workgroup dequantizes K into LDS as [key][d] and V as [d][key];
// each wave computes S^T = K Q^T (lane = query row, 16 keys per 32-key block), keeps an
// online softmax per row, and accumulates O^T += V^T P^T.  The P operand is taken in
// the key order the S^T accumulator already has, and V^T is read in that same order,
// so no register shuffle is needed between the two contractions.
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

__device__ __forceinline__ float q_at(const void* q, int dt, int64_t i) {
  if (dt == 0) return static_cast<const float*>(q)[i];
  const uint16_t b = static_cast<const uint16_t*>(q)[i];
  if (dt == 1) return __uint_as_float((uint32_t)b << 16);
  return h2f(b);
}

// Dequantize 8 consecutive elements whose codes start at byte `p` (fp16: values).
template <int BITS>
__device__ __forceinline__ void dequant8(const uint8_t* p, float d, _Float16 (&o)[8]) {
  if constexpr (BITS == 16) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xffffu));
      o[2 * i + 1] = __builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
    }
  } else if constexpr (BITS == 8) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    const uint32_t w[2] = {v.x, v.y};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = (int)(int8_t)((w[i >> 2] >> (8 * (i & 3))) & 0xff);
      o[i] = (_Float16)((float)c * d);   // exact product, one rounding to fp16
    }
  } else {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = (int)((w >> (4 * i)) & 0xf) - 8;
      o[i] = (_Float16)((float)c * d);
    }
  }
}

template <int KB, int VB, int D, bool QSPLIT>
__global__ __launch_bounds__(256, 2) void chunk_kernel(ChunkArgs a) {
  constexpr int NK = kChunkKeys;   // keys per tile
  constexpr int KSTR = D + 8;      // halves per LDS key row
  constexpr int VSTR = NK + 8;     // halves per LDS transposed-value row
  constexpr int NDT = D / 32;      // 32-wide output blocks along d
  constexpr int NKS = D / 16;      // k-steps of Q.K^T
  constexpr int KSEG = D / 8;      // 8-element segments per key row
  __shared__ __attribute__((aligned(16))) _Float16 s_k[NK * KSTR];
  __shared__ __attribute__((aligned(16))) _Float16 s_vt[D * VSTR];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, col = lane & 31;
  const int head = blockIdx.y, split = blockIdx.z;
  const int64_t rows = a.n_new * a.group;
  const int64_t tile_r0 = (int64_t)blockIdx.x * kChunkRows;
  const int64_t r0 = tile_r0 + wave * 32;
  const int64_t my_row = r0 + col;
  const bool valid = my_row < rows;
  const int64_t base_pos = a.len - a.n_new;
  const int64_t tok = valid ? my_row / a.group : 0;
  const int qh = head * a.group + (valid ? (int)(my_row % a.group) : 0);
  const int64_t pos = valid ? base_pos + tok : -1;

  const int64_t region = a.g.region();
  const uint8_t* kc = a.base + (int64_t)head * region;
  const uint8_t* ks = kc + a.g.off_ks();
  const uint8_t* vc = kc + a.g.off_vc();
  const uint8_t* vs = kc + a.g.off_vs();

  // Q^T as the B operand: lane (col, hl) holds d = 16 k + 8 hl .. + 7 of its row.
  // bf16 and fp16 queries are exact in fp16; fp32 queries are carried as hi + lo.
  half8_t qv[NKS];
  half8_t ql[QSPLIT ? NKS : 1];
  {
    const int64_t qoff = (tok * a.hq + qh) * (int64_t)D;
#pragma unroll
    for (int k = 0; k < NKS; ++k) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = valid ? q_at(a.q, a.q_dtype, qoff + 16 * k + 8 * hl + i) : 0.f;
        qv[k][i] = (_Float16)x;
        if constexpr (QSPLIT) ql[k][i] = (_Float16)(x - (float)qv[k][i]);
      }
    }
  }

  const int64_t k_lo = (int64_t)split * a.tps;
  const int64_t k_hi = min(k_lo + a.tps, a.len);
  const int64_t last_row = min(tile_r0 + kChunkRows, rows) - 1;
  const int64_t k_end = min(k_hi, base_pos + last_row / a.group + 1);
  const int64_t wave_min_pos = base_pos + r0 / a.group;
  const bool wave_active = r0 < rows;

  float m = -INFINITY, l = 0.f;
  float16_t o[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[t][v] = 0.f;

  for (int64_t kt0 = k_lo; kt0 < k_end; kt0 += NK) {
    // ---- K tile -> LDS [key][d] -------------------------------------------------
    for (int it = tid; it < NK * KSEG; it += 256) {
      const int t = it / KSEG, sg = it % KSEG;
      const int64_t key = kt0 + t;
      float d = 1.f;
      if constexpr (KB != 16) d = h2f(*reinterpret_cast<const uint16_t*>(ks + key * a.g.ks + 2 * (sg >> 2)));
      _Float16 v[8];
      dequant8<KB>(kc + key * a.g.kc + sg * KB, d, v);
      half8_t h;
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = v[i];
      *reinterpret_cast<half8_t*>(&s_k[t * KSTR + 8 * sg]) = h;
    }
    // ---- V tile -> LDS [d][key] (4 keys x 8 d per item) ---------------------------
    for (int it = tid; it < (NK / 4) * KSEG; it += 256) {
      const int kg = it % (NK / 4), sg = it / (NK / 4);
      _Float16 v[4][8];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int64_t key = kt0 + 4 * kg + kk;
        float d = 1.f;
        if constexpr (VB != 16) d = h2f(*reinterpret_cast<const uint16_t*>(vs + key * a.g.vs + 2 * (sg >> 2)));
        dequant8<VB>(vc + key * a.g.vc + sg * VB, d, v[kk]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        half4_t h;
        h[0] = v[0][e]; h[1] = v[1][e]; h[2] = v[2][e]; h[3] = v[3][e];
        *reinterpret_cast<half4_t*>(&s_vt[(8 * sg + e) * VSTR + 4 * kg]) = h;
      }
    }
    __syncthreads();

    if (wave_active) {
      // ---- S^T = K Q^T --------------------------------------------------------------
      float16_t s[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int v = 0; v < 16; ++v) s[st][v] = 0.f;
#pragma unroll
        for (int k = 0; k < NKS; ++k) {
          const half8_t ak = *reinterpret_cast<const half8_t*>(&s_k[(32 * st + col) * KSTR + 16 * k + 8 * hl]);
          s[st] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ak, qv[k], s[st], 0, 0, 0);
          if constexpr (QSPLIT) s[st] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ak, ql[k], s[st], 0, 0, 0);
        }
      }
      // ---- causal / range mask (only on tiles that reach the edge) ----------------
      if (kt0 + NK > k_end || kt0 + NK - 1 > wave_min_pos) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int64_t key = kt0 + 32 * st + 8 * (v >> 2) + 4 * hl + (v & 3);
            if (key >= k_end || key > pos) s[st][v] = -INFINITY;
          }
      }
      // ---- online softmax, one query row per lane pair (col, col + 32) ------------
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[st][v]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m, mx * a.qk_scale);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float alpha = __builtin_amdgcn_exp2f(m - mu);
      float ps = 0.f;
      half8_t pb[4];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[st][v], a.qk_scale, -mu));
          ps += p;
          pb[2 * st + (v >> 3)][v & 7] = (_Float16)p;
        }
      l = l * alpha + ps;
      m = mn;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int t = 0; t < NDT; ++t)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[t][v] *= alpha;
      }
      // ---- O^T += V^T P^T ---------------------------------------------------------------
#pragma unroll
      for (int t = 0; t < NDT; ++t) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const _Float16* vp = &s_vt[(32 * t + col) * VSTR + 32 * (kk >> 1) + 16 * (kk & 1) + 4 * hl];
          const half4_t lo = *reinterpret_cast<const half4_t*>(vp);
          const half4_t hi = *reinterpret_cast<const half4_t*>(vp + 8);
          half8_t av;
          av[0] = lo[0]; av[1] = lo[1]; av[2] = lo[2]; av[3] = lo[3];
          av[4] = hi[0]; av[5] = hi[1]; av[6] = hi[2]; av[7] = hi[3];
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, pb[kk], o[t], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  // ---- output -----------------------------------------------------------------------
  const float lt = l + __shfl_xor(l, 32);
  if (!valid) return;
  const int64_t orow = tok * a.hq + qh;
  if (a.n_splits == 1) {
    const float inv = 1.f / lt;
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * t + 8 * g4 + 4 * hl;
        float4 v = make_float4(o[t][4 * g4] * inv, o[t][4 * g4 + 1] * inv, o[t][4 * g4 + 2] * inv, o[t][4 * g4 + 3] * inv);
        *reinterpret_cast<float4*>(a.out + orow * D + d) = v;
      }
  } else {
    float* p = a.ws + (orow * a.n_splits + split) * (D + 2);
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * t + 8 * g4 + 4 * hl;
#pragma unroll
        for (int i = 0; i < 4; ++i) p[d + i] = o[t][4 * g4 + i];
      }
    if (hl == 0) {
      p[D] = m;
      p[D + 1] = lt;
    }
  }
}

template <int KB, int VB, int D>
hipError_t launch_t(const ChunkArgs& a, hipStream_t s) {
  const int64_t rows = a.n_new * a.group;
  const int64_t mt = (rows + kChunkRows - 1) / kChunkRows;
  dim3 grid((unsigned)mt, a.hkv, a.n_splits);
  if (a.q_dtype == 0)
    hipLaunchKernelGGL((chunk_kernel<KB, VB, D, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((chunk_kernel<KB, VB, D, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int KB, int VB>
hipError_t launch_d(const ChunkArgs& a, int d, hipStream_t s) {
  if (d == 64) return launch_t<KB, VB, 64>(a, s);
  if (d == 128) return launch_t<KB, VB, 128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_chunk(const ChunkArgs& a, int kbits, int vbits, int d, hipStream_t s) {
  if (kbits == 16 && vbits == 16) return launch_d<16, 16>(a, d, s);
  if (kbits == 8 && vbits == 8) return launch_d<8, 8>(a, d, s);
  if (kbits == 8 && vbits == 4) return launch_d<8, 4>(a, d, s);
  if (kbits == 4 && vbits == 8) return launch_d<4, 8>(a, d, s);
  if (kbits == 4 && vbits == 4) return launch_d<4, 4>(a, d, s);
  return hipErrorInvalidValue;
}

}  // namespace kvq

// Single-query (decode) attention over the packed session cache, split along the
// context.  Attention is softmax(sigma q.K^T) V over the dequantized cache; keys and
// values keep their own bit widths ("KVSplit -- contexto 2 a 3 vezes mais longo em
// Apple Silicon", sections "Principais resultados de benchmark" and "Assimetria entre
// key e value").  The same page's discussion ("Opinioes no Hacker News") places the
// gain in memory traffic, and the openclawradar.com page ("O Que Nao Funcionou") saw
// 8-bit KV lose throughput when dequantization cost more than the bytes it saved, so
// codes are dequantized in registers, never materialized.
//
// Work split: one workgroup (4 waves) per (split of the context, KV head, session);
// each wave takes 128-token chunks of the split in turn.  Within a wave, E = D / LPT
// elements of a token belong to one lane (LPT lanes per token), and each lane holds
// two tokens per step, t and t + 64 / LPT.  A chunk is processed in three phases:
//   A  scores: integer dot products (v_dot4_i32_i8) of the 8/4-bit key codes with the
//      query split into two int8 digits, or fp16 dot2 for the fp16 control; partial
//      sums are reduced over the LPT lanes with DPP;
//   B  one lane per token: exact running max of the chunk per query head, p = 2^(s-m),
//      the accumulators rescaled only when the max moved;
//   C  values: v_dot2_f32_f16 over the token pair with weights w = p*d in fp16 and
//      the value codes laid into fp16 subnormal bit patterns (u * 2^-24), so that no
//      large bias enters the fp32 accumulators.
// The epilogue reduces the wave's partials, merges the four waves through LDS, and
// writes either the normalized output (one split) or (o, m, l) for the merge kernel.
#include "kvq_internal.h"
#include "wave_ops.h"

namespace kvq {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half2_t as_h2(uint32_t x) { return __builtin_bit_cast(half2_t, x); }
__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ __forceinline__ half2_t pack_rne(float a, float b) {
  half2_t r;
  r.x = (_Float16)a;
  r.y = (_Float16)b;
  return r;
}

template <int W>
__device__ __forceinline__ void load_dwords(const uint8_t* p, uint32_t (&o)[W]) {
  if constexpr (W % 4 == 0) {
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      uint4 t = reinterpret_cast<const uint4*>(p)[i];
      o[4 * i] = t.x; o[4 * i + 1] = t.y; o[4 * i + 2] = t.z; o[4 * i + 3] = t.w;
    }
  } else if constexpr (W == 2) {
    uint2 t = *reinterpret_cast<const uint2*>(p);
    o[0] = t.x; o[1] = t.y;
  } else {
    static_assert(W == 1, "dword count");
    o[0] = *reinterpret_cast<const uint32_t*>(p);
  }
}

__device__ __forceinline__ float load_q(const void* q, int dt, int64_t i) {
  if (dt == 0) return static_cast<const float*>(q)[i];
  uint16_t b = static_cast<const uint16_t*>(q)[i];
  if (dt == 1) return __uint_as_float((uint32_t)b << 16);
  return h2f(b);
}

template <int KB, int VB, int D, int GP, int E>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  constexpr int LPT = D / E;           // lanes per token
  constexpr int TPS = 64 / LPT;        // tokens per half step
  constexpr int STEP = 2 * TPS;        // tokens per step (two per lane)
  constexpr int CT = kDecodeChunk;     // tokens per chunk
  constexpr int NS = CT / STEP;        // steps per chunk
  constexpr int NB = D / kBlock;       // blocks per row
  constexpr int KW = KB == 16 ? E / 2 : (KB == 8 ? E / 4 : E / 8);  // key dwords per token per lane
  constexpr int VW = VB == 16 ? E / 2 : (VB == 8 ? E / 4 : E / 8);  // value dwords per token per lane
  constexpr int QW = KB == 16 ? E / 2 : E / 4;                       // query dwords per head
  static_assert(E <= kBlock && kBlock % E == 0, "a lane stays inside one block");
  static_assert(CT % STEP == 0 && CT == 128, "chunk shape");

  __shared__ float s_q[GP][D];
  __shared__ float s_qs[GP][NB];
  __shared__ __attribute__((aligned(16))) int8_t s_qa[GP][D];
  __shared__ __attribute__((aligned(16))) int8_t s_qb[GP][D];
  __shared__ float s_sc[4][CT][GP];
  __shared__ float s_o[4][GP][D];
  __shared__ float s_ml[4][2][GP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, head = blockIdx.y, sl = blockIdx.z;
  const SessionRef S = a.sess[sl];
  const int64_t srow = (int64_t)(a.sess0 + sl) * a.hq + (int64_t)head * a.group;  // first q row
  const int64_t ts = (int64_t)split * a.tps;
  const int64_t te = min(ts + a.tps, S.len);
  const int64_t region = S.cap * (int64_t)(a.kc + a.ks + a.vc + a.vs);
  const uint8_t* kc = S.base + (int64_t)head * region;
  const uint8_t* ks = kc + S.cap * a.kc;
  const uint8_t* vc = ks + S.cap * a.ks;
  const uint8_t* vs = vc + S.cap * a.vc;

  // ---- query preparation: fp32 copy, then per (head, block) two int8 digits -------
  for (int i = tid; i < GP * D; i += 256) {
    int g = i / D, e = i % D;
    s_q[g][e] = g < a.group ? load_q(a.q, a.q_dtype, (srow + g) * D + e) : 0.f;
  }
  __syncthreads();
  if (tid < GP * NB) {
    const int g = tid / NB, b = tid % NB;
    if constexpr (KB == 16) {
      s_qs[g][b] = a.qk_scale;
    } else {
      float amax = 0.f;
      for (int e = 0; e < kBlock; ++e) amax = fmaxf(amax, fabsf(s_q[g][b * kBlock + e]));
      // q ~= sq * (256 * qa + qb), |qa| <= 127, qb in [-128, 127]
      const float sq = amax / 32512.f;
      for (int e = 0; e < kBlock; ++e) {
        float v = sq > 0.f ? rintf(s_q[g][b * kBlock + e] / sq) : 0.f;
        v = fminf(fmaxf(v, -32512.f), 32512.f);
        int Q = (int)v;
        int qa = (Q + 128) >> 8;  // floor((Q + 128) / 256)
        s_qa[g][b * kBlock + e] = (int8_t)qa;
        s_qb[g][b * kBlock + e] = (int8_t)(Q - 256 * qa);
      }
      s_qs[g][b] = sq * a.qk_scale;
    }
  }
  __syncthreads();

  const int sub = lane % LPT, grp = lane / LPT, e0 = sub * E, blk = e0 / kBlock;
  uint32_t qa_r[GP][QW], qb_r[GP][QW];
  int corr_a[GP], corr_b[GP];
  float qsc[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    qsc[g] = s_qs[g][blk];
    corr_a[g] = 0;
    corr_b[g] = 0;
    if constexpr (KB == 16) {
#pragma unroll
      for (int j = 0; j < QW; ++j)
        qa_r[g][j] = __builtin_bit_cast(uint32_t, pack_rne(s_q[g][e0 + 2 * j], s_q[g][e0 + 2 * j + 1]));
    } else if constexpr (KB == 8) {
#pragma unroll
      for (int j = 0; j < QW; ++j) {
        qa_r[g][j] = *reinterpret_cast<const uint32_t*>(&s_qa[g][e0 + 4 * j]);
        qb_r[g][j] = *reinterpret_cast<const uint32_t*>(&s_qb[g][e0 + 4 * j]);
      }
    } else {
      // 4-bit keys: a code dword covers 8 elements; its low nibbles are the even ones
#pragma unroll
      for (int j = 0; j < E / 8; ++j) {
        uint32_t ae = 0, ao = 0, be = 0, bo = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          ae |= (uint32_t)(uint8_t)s_qa[g][e0 + 8 * j + 2 * k] << (8 * k);
          ao |= (uint32_t)(uint8_t)s_qa[g][e0 + 8 * j + 2 * k + 1] << (8 * k);
          be |= (uint32_t)(uint8_t)s_qb[g][e0 + 8 * j + 2 * k] << (8 * k);
          bo |= (uint32_t)(uint8_t)s_qb[g][e0 + 8 * j + 2 * k + 1] << (8 * k);
        }
        qa_r[g][2 * j] = ae; qa_r[g][2 * j + 1] = ao;
        qb_r[g][2 * j] = be; qb_r[g][2 * j + 1] = bo;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        corr_a[g] -= 8 * s_qa[g][e0 + e];
        corr_b[g] -= 8 * s_qb[g][e0 + e];
      }
    }
  }

  float acc[GP][E];
  float wsum[GP], lsum[GP], m[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    wsum[g] = 0.f;
    lsum[g] = 0.f;
    m[g] = -INFINITY;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[g][e] = 0.f;
  }

  const uint32_t koff = grp * a.kc + sub * (KW * 4), ksoff = grp * a.ks + blk * 2;
  const uint32_t voff = grp * a.vc + sub * (VW * 4), vsoff = grp * a.vs + blk * 2;
  const int64_t n_chunks = te > ts ? (te - ts + CT - 1) / CT : 0;
  for (int64_t c = __builtin_amdgcn_readfirstlane(wave); c < n_chunks; c += 4) {
    const int64_t c0 = ts + c * CT;
    // wave-uniform chunk bases; per-lane offsets inside a chunk fit 32 bits
    const uint8_t* kcc = kc + c0 * a.kc;
    const uint8_t* ksc = ks + c0 * a.ks;
    const uint8_t* vcc = vc + c0 * a.vc;
    const uint8_t* vsc = vs + c0 * a.vs;
    const bool tail = c0 + CT > te;
    // ---- phase A: scores (codes of step s + 1 in flight while step s computes) ----
    uint32_t kbuf[2][2][KW];
    uint16_t kscl[2][2] = {{0, 0}, {0, 0}};
    // address = uniform base (chunk, step, token half) + one loop-invariant lane offset
    auto load_k = [&](int s, int slot) {
      const uint8_t* c0p = kcc + (int64_t)(s * STEP) * a.kc;
      load_dwords<KW>(c0p + koff, kbuf[slot][0]);
      load_dwords<KW>(c0p + (int64_t)TPS * a.kc + koff, kbuf[slot][1]);
      if constexpr (KB != 16) {
        const uint8_t* s0p = ksc + (int64_t)(s * STEP) * a.ks;
        kscl[slot][0] = *reinterpret_cast<const uint16_t*>(s0p + ksoff);
        kscl[slot][1] = *reinterpret_cast<const uint16_t*>(s0p + (int64_t)TPS * a.ks + ksoff);
      }
    };
    load_k(0, 0);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int la = s * STEP + grp, lb = la + TPS;
      if (s + 1 < NS) load_k(s + 1, (s + 1) & 1);
      const uint32_t* ka = kbuf[s & 1][0];
      const uint32_t* kb = kbuf[s & 1][1];
      float da = 1.f, db = 1.f;
      if constexpr (KB != 16) {
        da = h2f(kscl[s & 1][0]);
        db = h2f(kscl[s & 1][1]);
      }
      float pa[GP], pb[GP];
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        if constexpr (KB == 16) {
          float xa = 0.f, xb = 0.f;
#pragma unroll
          for (int j = 0; j < KW; ++j) {
            xa = __builtin_amdgcn_fdot2(as_h2(qa_r[g][j]), as_h2(ka[j]), xa, false);
            xb = __builtin_amdgcn_fdot2(as_h2(qa_r[g][j]), as_h2(kb[j]), xb, false);
          }
          pa[g] = xa * qsc[g];
          pb[g] = xb * qsc[g];
        } else {
          // one chain per token: high digit, times 256, then the low digit
          int ha = corr_a[g], hb = corr_a[g];
          if constexpr (KB == 8) {
#pragma unroll
            for (int j = 0; j < KW; ++j) {
              ha = __builtin_amdgcn_sdot4((int)ka[j], (int)qa_r[g][j], ha, false);
              hb = __builtin_amdgcn_sdot4((int)kb[j], (int)qa_r[g][j], hb, false);
            }
            ha = (ha << 8) + corr_b[g];
            hb = (hb << 8) + corr_b[g];
#pragma unroll
            for (int j = 0; j < KW; ++j) {
              ha = __builtin_amdgcn_sdot4((int)ka[j], (int)qb_r[g][j], ha, false);
              hb = __builtin_amdgcn_sdot4((int)kb[j], (int)qb_r[g][j], hb, false);
            }
          } else {
            uint32_t ae[KW], ao[KW], be[KW], bo[KW];
#pragma unroll
            for (int j = 0; j < KW; ++j) {
              ae[j] = ka[j] & 0x0F0F0F0Fu; ao[j] = (ka[j] >> 4) & 0x0F0F0F0Fu;
              be[j] = kb[j] & 0x0F0F0F0Fu; bo[j] = (kb[j] >> 4) & 0x0F0F0F0Fu;
            }
#pragma unroll
            for (int j = 0; j < KW; ++j) {
              ha = __builtin_amdgcn_sdot4((int)ae[j], (int)qa_r[g][2 * j], ha, false);
              ha = __builtin_amdgcn_sdot4((int)ao[j], (int)qa_r[g][2 * j + 1], ha, false);
              hb = __builtin_amdgcn_sdot4((int)be[j], (int)qa_r[g][2 * j], hb, false);
              hb = __builtin_amdgcn_sdot4((int)bo[j], (int)qa_r[g][2 * j + 1], hb, false);
            }
            ha = (ha << 8) + corr_b[g];
            hb = (hb << 8) + corr_b[g];
#pragma unroll
            for (int j = 0; j < KW; ++j) {
              ha = __builtin_amdgcn_sdot4((int)ae[j], (int)qb_r[g][2 * j], ha, false);
              ha = __builtin_amdgcn_sdot4((int)ao[j], (int)qb_r[g][2 * j + 1], ha, false);
              hb = __builtin_amdgcn_sdot4((int)be[j], (int)qb_r[g][2 * j], hb, false);
              hb = __builtin_amdgcn_sdot4((int)bo[j], (int)qb_r[g][2 * j + 1], hb, false);
            }
          }
          pa[g] = (float)ha * (da * qsc[g]);
          pb[g] = (float)hb * (db * qsc[g]);
        }
        pa[g] = group_sum<LPT>(pa[g]);
        pb[g] = group_sum<LPT>(pb[g]);
      }
      if (sub == 0) {
#pragma unroll
        for (int g = 0; g < GP; ++g) {
          s_sc[wave][la][g] = pa[g];
          s_sc[wave][lb][g] = pb[g];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the first value codes of the chunk fly during the softmax statistics
    uint32_t vbuf[2][2][VW];
    uint16_t vscl[2][2] = {{0, 0}, {0, 0}};
    auto load_v = [&](int s, int slot) {
      const uint8_t* c0p = vcc + (int64_t)(s * STEP) * a.vc;
      load_dwords<VW>(c0p + voff, vbuf[slot][0]);
      load_dwords<VW>(c0p + (int64_t)TPS * a.vc + voff, vbuf[slot][1]);
      if constexpr (VB != 16) {
        const uint8_t* s0p = vsc + (int64_t)(s * STEP) * a.vs;
        vscl[slot][0] = *reinterpret_cast<const uint16_t*>(s0p + vsoff);
        vscl[slot][1] = *reinterpret_cast<const uint16_t*>(s0p + (int64_t)TPS * a.vs + vsoff);
      }
    };
    load_v(0, 0);
    wave_lds_sync();
    // ---- phase B: softmax statistics, one lane per token ------------------------
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      float sa = s_sc[wave][lane][g], sb = s_sc[wave][lane + 64][g];
      if (tail) {  // tokens past the cached length score -inf
        if (c0 + lane >= te) sa = -INFINITY;
        if (c0 + lane + 64 >= te) sb = -INFINITY;
      }
      const float cm = wave_max(fmaxf(sa, sb));
      const float mn = fmaxf(m[g], cm);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float alpha = __builtin_amdgcn_exp2f(m[g] - mu);
      const float p0 = __builtin_amdgcn_exp2f(sa - mu), p1 = __builtin_amdgcn_exp2f(sb - mu);
      s_sc[wave][lane][g] = p0;
      s_sc[wave][lane + 64][g] = p1;
      lsum[g] = lsum[g] * alpha + (p0 + p1);
      if (alpha != 1.f) {  // wave-uniform
#pragma unroll
        for (int e = 0; e < E; ++e) acc[g][e] *= alpha;
        wsum[g] *= alpha;
      }
      m[g] = mn;
    }
    wave_lds_sync();
    // ---- phase C: values (codes of step s + 1 in flight while step s computes) ---
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int la = s * STEP + grp, lb = la + TPS;
      if (s + 1 < NS) load_v(s + 1, (s + 1) & 1);
      const uint32_t* va = vbuf[s & 1][0];
      const uint32_t* vb = vbuf[s & 1][1];
      float da = 1.f, db = 1.f;
      if constexpr (VB != 16) {
        da = h2f(vscl[s & 1][0]);
        db = h2f(vscl[s & 1][1]);
      }
      half2_t w[GP];
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        w[g] = pack_rne(s_sc[wave][la][g] * da, s_sc[wave][lb][g] * db);
        wsum[g] = __builtin_amdgcn_fdot2(w[g], as_h2(0x3C003C00u), wsum[g], false);
      }
#pragma unroll
      for (int j = 0; j < VW; ++j) {
        if constexpr (VB == 4) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t sel = (uint32_t)k | (0x0cu << 8) | ((uint32_t)(4 + k) << 16) | (0x0cu << 24);
            const uint32_t pr = __builtin_amdgcn_perm(vb[j], va[j], sel);
            const half2_t ev = as_h2(pr & 0x000F000Fu), od = as_h2(pr & 0x00F000F0u);
#pragma unroll
            for (int g = 0; g < GP; ++g) {
              acc[g][8 * j + 2 * k] = __builtin_amdgcn_fdot2(w[g], ev, acc[g][8 * j + 2 * k], false);
              acc[g][8 * j + 2 * k + 1] = __builtin_amdgcn_fdot2(w[g], od, acc[g][8 * j + 2 * k + 1], false);
            }
          }
        } else if constexpr (VB == 8) {
          const uint32_t xa = va[j] ^ 0x80808080u, xb = vb[j] ^ 0x80808080u;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t sel = (uint32_t)k | (0x0cu << 8) | ((uint32_t)(4 + k) << 16) | (0x0cu << 24);
            const half2_t pr = as_h2(__builtin_amdgcn_perm(xb, xa, sel));
#pragma unroll
            for (int g = 0; g < GP; ++g)
              acc[g][4 * j + k] = __builtin_amdgcn_fdot2(w[g], pr, acc[g][4 * j + k], false);
          }
        } else {
          const half2_t p0 = as_h2(__builtin_amdgcn_perm(vb[j], va[j], 0x05040100u));
          const half2_t p1 = as_h2(__builtin_amdgcn_perm(vb[j], va[j], 0x07060302u));
#pragma unroll
          for (int g = 0; g < GP; ++g) {
            acc[g][2 * j] = __builtin_amdgcn_fdot2(w[g], p0, acc[g][2 * j], false);
            acc[g][2 * j + 1] = __builtin_amdgcn_fdot2(w[g], p1, acc[g][2 * j + 1], false);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    wave_lds_sync();
  }

  // ---- epilogue: wave partials -> workgroup partial -------------------------------
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    const float lw = wave_sum(lsum[g]);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float o;
      if constexpr (VB == 4) o = acc[g][e] * ((e & 1) ? 1048576.f : 16777216.f) - 8.f * wsum[g];
      else if constexpr (VB == 8) o = acc[g][e] * 16777216.f - 128.f * wsum[g];
      else o = acc[g][e];
      o = strided_sum<LPT>(o);
      if (grp == 0) s_o[wave][g][e0 + e] = o;
    }
    if (lane == 0) {
      s_ml[wave][0][g] = m[g];
      s_ml[wave][1][g] = lw;
    }
  }
  __syncthreads();
  for (int i = tid; i < GP * D; i += 256) {
    const int g = i / D, e = i % D;
    if (g >= a.group) continue;
    float mw[4], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      mw[w] = s_ml[w][0][g];
      M = fmaxf(M, mw[w]);
    }
    float o = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = mw[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[w] - M);
        o += f * s_o[w][g][e];
        l += f * s_ml[w][1][g];
      }
    }
    const int64_t row = srow + g;
    if (!a.partial) {
      a.out[row * D + e] = o / l;
    } else {
      float* p = a.ws + (row * a.n_splits + split) * (D + 2);
      p[e] = o;
      if (e == 0) {
        p[D] = M;
        p[D + 1] = l;
      }
    }
  }
}

template <int GP>
constexpr int lane_elems() { return GP <= 2 ? 32 : (GP == 4 ? 16 : 8); }

template <int KB, int VB, int D, int GP>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
  constexpr int E = lane_elems<GP>();
  dim3 grid(a.n_splits, a.hkv, a.n_sess);
  hipLaunchKernelGGL((decode_kernel<KB, VB, D, GP, E>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int KB, int VB, int D>
hipError_t launch_g(const DecodeArgs& a, int gp, hipStream_t s) {
  switch (gp) {
    case 1: return launch_t<KB, VB, D, 1>(a, s);
    case 2: return launch_t<KB, VB, D, 2>(a, s);
    case 4: return launch_t<KB, VB, D, 4>(a, s);
    case 8: return launch_t<KB, VB, D, 8>(a, s);
    case 16: return launch_t<KB, VB, D, 16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int KB, int VB>
hipError_t launch_d(const DecodeArgs& a, int d, int gp, hipStream_t s) {
  if (d == 64) return launch_g<KB, VB, 64>(a, gp, s);
  if (d == 128) return launch_g<KB, VB, 128>(a, gp, s);
  return hipErrorInvalidValue;
}

template <int KB, int VB, int D>
const void* ptr_g(int gp) {
  switch (gp) {
    case 1: return reinterpret_cast<const void*>(&decode_kernel<KB, VB, D, 1, lane_elems<1>()>);
    case 2: return reinterpret_cast<const void*>(&decode_kernel<KB, VB, D, 2, lane_elems<2>()>);
    case 4: return reinterpret_cast<const void*>(&decode_kernel<KB, VB, D, 4, lane_elems<4>()>);
    case 8: return reinterpret_cast<const void*>(&decode_kernel<KB, VB, D, 8, lane_elems<8>()>);
    default: return reinterpret_cast<const void*>(&decode_kernel<KB, VB, D, 16, lane_elems<16>()>);
  }
}

template <int KB, int VB>
const void* ptr_d(int d, int gp) {
  return d == 64 ? ptr_g<KB, VB, 64>(gp) : ptr_g<KB, VB, 128>(gp);
}

}  // namespace

const void* decode_kernel_for(int kbits, int vbits, int d, int gp) {
  if (kbits == 16) return ptr_d<16, 16>(d, gp);
  if (kbits == 8 && vbits == 8) return ptr_d<8, 8>(d, gp);
  if (kbits == 8) return ptr_d<8, 4>(d, gp);
  if (vbits == 8) return ptr_d<4, 8>(d, gp);
  return ptr_d<4, 4>(d, gp);
}

hipError_t launch_decode(const DecodeArgs& a, int kbits, int vbits, int d, int gp, hipStream_t s) {
  if (kbits == 16 && vbits == 16) return launch_d<16, 16>(a, d, gp, s);
  if (kbits == 8 && vbits == 8) return launch_d<8, 8>(a, d, gp, s);
  if (kbits == 8 && vbits == 4) return launch_d<8, 4>(a, d, gp, s);
  if (kbits == 4 && vbits == 8) return launch_d<4, 8>(a, d, gp, s);
  if (kbits == 4 && vbits == 4) return launch_d<4, 4>(a, d, gp, s);
  return hipErrorInvalidValue;
}

}  // namespace kvq

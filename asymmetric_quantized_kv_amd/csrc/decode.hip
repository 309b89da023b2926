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
// each wave takes 128-token chunks of the split in turn.  The grid runs KV head fastest,
// then session, then split: the runtime deals workgroups to the 8 XCDs round-robin by
// linear id, so each die gets the same heads of every session (equal work), and the splits
// that are empty for short sessions come last.  (Split fastest would put every workgroup
// of split s on die s whenever the split count is a multiple of 8.)  Within a wave, E = D / LPT
// elements of a token belong to one lane (LPT lanes per token), and each lane holds
// two tokens per step, t and t + 64 / LPT.  A chunk is processed in three phases:
//   A  scores, on the matrix cores for quantized keys: the query (one scale per head)
//      split into two int8 digits meets 32 tokens' 8/4-bit key codes of one 32-element
//      block in v_mfma_i32_32x32x32_i8 (exact integer block sums, then the block's d);
//      fp8 (E4M3) key codes are widened to fp16 with the block's power-of-two scale folded
//      into the conversion (exact) and meet the query (scaled by a power of two into
//      fp16's range, fp32 queries as fp16 hi + lo) in v_mfma_f32_32x32x16_f16.  The fp16
//      control, and 4-bit keys at group 16, use VALU dot products (fp16 dot2, v_dot4) with
//      the lanes of a token reduced by DPP;
//   B  one lane per token: the query's scale turns the raw score into a base-2 logit;
//      exact running max of the chunk per query head, p = 2^(s-m),
//      the accumulators rescaled only when the max moved;
//   C  values: v_dot2_f32_f16 over the token pair with weights w = p*d in fp16 and
//      the value codes laid into fp16 subnormal bit patterns (u * 2^-24), so that no
//      large bias enters the fp32 accumulators.
// The epilogue reduces the wave's partials, merges the four waves through LDS, and
// writes either the normalized output (one split) or (o, m, l) for the merge kernel.
#include "kvq_internal.h"
#include "buffer_ops.h"
#include "wave_ops.h"
#include "merge_row.h"

constexpr int kDecodeDepth = 4;   // steps of key/value codes requested ahead of the one computing

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

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// a . b over four signed bytes, starting a new sum (the VOP3 form takes the zero as an
// inline constant; the accumulating two-operand form would need a register cleared first)
__device__ __forceinline__ int sdot4_start(int a, int b) {
  int r;
  asm("v_dot4_i32_i8 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Integer sum over aligned groups of N consecutive lanes (N = 1, 2, 4).
template <int N>
__device__ __forceinline__ int group_sum_i(int x) {
  if constexpr (N >= 2) x += __builtin_amdgcn_mov_dpp(x, kDppXor1, 0xf, 0xf, true);
  if constexpr (N >= 4) x += __builtin_amdgcn_mov_dpp(x, kDppXor2, 0xf, 0xf, true);
  return x;
}

// Float sum over groups of N lanes that are NI-aligned and already hold the sum of
// their NI-lane subgroup (NI | N; N <= 16).
template <int N, int NI>
__device__ __forceinline__ float group_sum_rest(float x) {
  if constexpr (NI < 2 && N >= 2) x += dpp<kDppXor1>(x);
  if constexpr (NI < 4 && N >= 4) x += dpp<kDppXor2>(x);
  if constexpr (NI < 8 && N >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (NI < 16 && N >= 16) x += dpp<kDppMirror>(x);
  return x;
}

__device__ __forceinline__ float load_q(const void* q, int dt, int64_t i) {
  if (dt == 0) return static_cast<const float*>(q)[i];
  uint16_t b = static_cast<const uint16_t*>(q)[i];
  if (dt == 1) return __uint_as_float((uint32_t)b << 16);
  return h2f(b);
}

// A fused split launch: every workgroup writes its partial (o, m, l) with agent-scope atomic
// stores and then counts itself on its session's counter for the KV head; the one that brings
// the count to the number of splits reads all of them back with agent-scope atomic loads and
// writes the merged rows (out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, M = max_s m_s;
// splits with m = -inf drop out), then leaves the counter at zero for the next call.
// Agent-scope atomic accesses are coherent across the XCDs' separate L2 caches on their own
// (stores write through, loads read past this L2's lines); a workgroup counts only after its
// stores have completed (vmcnt(0) ahead of the barrier), and the last one loads only after its
// count has returned.  That takes the place of a release and an acquire fence, each of which
// writes back or invalidates the whole L2 here.  One lane does the count, as a vector atomic.
// A partial's word: an agent-scope atomic store (written through past this XCD's L2), so the
// merging workgroup of the same launch can read it on any XCD.
__device__ __forceinline__ void st_partial(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D>
__device__ void merge_if_last(const DecodeArgs& a, const SessionRef& S, int n_s, int64_t srow, int head, int tid,
                              int* s_last) {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this lane's partial stores have completed
  __syncthreads();
  if (tid == 0) {
    const uint32_t before = __hip_atomic_fetch_add(S.counters + head, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = before + 1u == (uint32_t)n_s;
    if (last) __hip_atomic_store(S.counters + head, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_last = last;
  }
  __syncthreads();
  if (!*s_last) return;
  // the same row merge as the standalone merge kernels would run under this plan
  const float* p0 = a.ws + srow * a.n_splits * (int64_t)(D + 2);
  float* o0 = a.out + srow * D;
  if (merge_seq_form(D, a.n_splits)) {
    constexpr int LPR = D / 8;
    for (int i = tid; i < a.group * LPR; i += 256)
      merge_row_seq<D, true>(p0 + (i / LPR) * a.n_splits * (int64_t)(D + 2), n_s, i % LPR, o0 + (i / LPR) * D);
  } else {
    for (int g = tid >> 6; g < a.group; g += 4)   // a wave per row, every lane active
      merge_row_wave<true>(p0 + g * a.n_splits * (int64_t)(D + 2), n_s, D, o0 + g * D, tid & 63);
  }
}

// QLO: fp8 or fp16 keys with fp32 queries, which carry an fp16 low part (16-bit queries are
// exact in fp16 after the power-of-two prescale)
// ONE: every wave holds at most one chunk (a split of at most 4 x 128 tokens): all of its key
// and value codes are requested before the query is prepared, so a small launch pays one
// memory latency instead of a chain of them.
// STREAM: a streamed launch (DecodeArgs::stream), each workgroup taking in turn the part of
// every session its block range overlaps
template <int KB, int VB, int D, int GP, int E, bool QLO = false, bool ONE = false, bool STREAM = false>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  constexpr int LPT = D / E;           // lanes per token
  constexpr int TPS = 64 / LPT;        // tokens per half step
  constexpr int STEP = 2 * TPS;        // tokens per step (two per lane)
  constexpr int CT = kDecodeChunk;     // tokens per chunk
  constexpr int NS = CT / STEP;        // steps per chunk
  constexpr int NB = D / kBlock;       // blocks per row
  constexpr int KW = KB == 16 ? E / 2 : (KB == 4 ? E / 8 : E / 4);  // key dwords per token per lane
  constexpr int VW = VB == 16 ? E / 2 : (VB == 8 ? E / 4 : E / 8);  // value dwords per token per lane
  constexpr int QW = KB == 16 || KB == kF8 ? E / 2 : E / 4;         // query dwords per head
  constexpr int KC = code_row_bytes(KB, D), KS = scale_row_bytes(KB, D);  // row bytes per plane
  constexpr int VC = code_row_bytes(VB, D), VS = scale_row_bytes(VB, D);
  constexpr int LPB = kBlock / E;      // lanes per block (their key codes share one scale)
  static_assert(E <= kBlock && kBlock % E == 0, "a lane stays inside one block");
  static_assert(CT % STEP == 0 && CT == 128, "chunk shape");

  __shared__ float s_q[GP][D];
  __shared__ float s_qs[GP];
  __shared__ float s_qi[GP];                               // fp8 / fp16 keys: power-of-two query prescale
  __shared__ __attribute__((aligned(16))) int8_t s_qa[GP][D];
  __shared__ __attribute__((aligned(16))) int8_t s_qb[GP][D];
  __shared__ float s_sc[4][CT][GP];                        // raw scores of a chunk
  __shared__ __attribute__((aligned(16))) uint32_t s_w[4][CT / 2][GP];  // fp16 p of token pairs
  __shared__ float s_o[4][GP][D];
  __shared__ float s_ml[4][2][GP];
  __shared__ int s_last;                                   // fused launches: this workgroup merges

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int vhead = blockIdx.x, head = vhead / a.hsplit;   // the workgroup's part of KV head `head`
  // streamed launches: blocks [blk, blk_end) of the sessions' blocks laid end to end
  int64_t blk = 0, blk_end = 0;
  if constexpr (STREAM) {
    blk = a.wg_block0[blockIdx.y];
    blk_end = a.wg_block0[blockIdx.y + 1];
    if (blk >= blk_end) return;
  }
  do {   // once, or (streamed) once per session the block range overlaps
  SessionRef S;
  int split, n_merge;   // the partial's index among the session's, and their number
  int64_t ts, te;       // the session's tokens [ts, te) taken here
  bool part;            // write a partial (else the normalized output)
  if constexpr (STREAM) {
    int lo = 0, hi = a.n_sess - 1;   // the last session whose first block is at or before blk
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.sess[mid].piece0 <= blk) lo = mid; else hi = mid - 1;
    }
    S = a.sess[lo];
    const int64_t first = S.piece0, nb = (S.len + kDecodeWaveTokens - 1) / kDecodeWaveTokens;
    const int64_t b1 = min(blk_end, first + nb);
    ts = (blk - first) * kDecodeWaveTokens;
    te = min(S.len, (b1 - first) * kDecodeWaveTokens);
    split = (int)blockIdx.y - S.wfirst;
    n_merge = S.nseg;
    part = S.nseg > 1;
    blk = b1;
  } else {
    int sl = blockIdx.y;
    split = blockIdx.z;
    // the full grid's session, read before the launch kind is known (no wait on a.compact
    // first: the empty asm keeps the compiler from sinking these loads past the branch)
    S = a.sess[min(sl, kMaxSessions - 1)];
    asm volatile("" : "+s"(S.base), "+s"(S.cap), "+s"(S.len));
    if (a.compact) {   // blockIdx.y enumerates the busy (session, split) pairs: the last session
      int lo = 0, hi = a.n_sess - 1;   // whose first piece is at or before it
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.sess[mid].piece0 <= sl) lo = mid; else hi = mid - 1;
      }
      split = sl - a.sess[lo].piece0;
      sl = lo;
      S = a.sess[sl];
    }
    ts = (int64_t)split * a.tps;
    te = min(ts + a.tps, S.len);
    n_merge = a.compact ? (int)((S.len + a.tps - 1) / a.tps) : a.n_splits;
    part = a.partial;
  }
  const int64_t srow = S.row * a.hq + (int64_t)vhead * a.group;  // first q row
  if (ts >= S.len) {
    // a split past this session's end (shorter sessions in a batch): an empty partial
    if (part) {
      for (int i = tid; i < a.group * (D + 2); i += 256) {
        const int g = i / (D + 2), e = i % (D + 2);
        st_partial(a.ws + ((srow + g) * a.n_splits + split) * (D + 2) + e, e == D ? -INFINITY : 0.f);
      }
      if (a.fused) merge_if_last<D>(a, S, n_merge, srow, vhead, tid, &s_last);
    }
    return;
  }
  const int64_t region = S.cap * (int64_t)(KC + KS + VC + VS);
  const uint8_t* kc = S.base + (int64_t)head * region;
  const uint8_t* ks = kc + S.cap * KC;
  const uint8_t* vc = ks + S.cap * KS;
  const uint8_t* vs = vc + S.cap * VC;

  const int sub = lane % LPT, grp = lane / LPT, e0 = sub * E, blk = e0 / kBlock;
  // Q.K on the matrix cores: 8/4-bit keys (int8 MFMA per 32-element block; 4-bit keys at group
  // 16 keep the VALU path) and fp8 keys (fp16 MFMA over the widened keys)
  constexpr bool MQK = KB == 8 || (KB == 4 && GP <= 8);
  constexpr bool MQF = KB == kF8;
  constexpr bool MQ = MQK || MQF;

  // ---- the first key (and, for ONE, value) codes go out before the query is prepared ------
  const uint32_t koff = grp * KC + sub * (KW * 4), ksoff = grp * KS + blk * (KB == kF8 ? 1 : 2);
  const uint32_t voff = grp * VC + sub * (VW * 4), vsoff = grp * VS + blk * 2;
  const int64_t n_chunks = te > ts ? (te - ts + CT - 1) / CT : 0;
  // Load pipeline: step s of a phase uses ring slot s % R, and the codes of the step
  // PD steps ahead are requested before step s computes.  The last PD steps of phase A
  // request the first value steps of the chunk, and the last PD steps of phase C the
  // first key steps of the wave's next chunk, so the pipeline never drains.
  constexpr int PD = ONE ? NS : (kDecodeDepth < NS ? kDecodeDepth : NS - 1), R = ONE ? NS : PD + 1;
  static_assert(PD >= 1, "prefetch depth");
  uint32_t kbuf[R][2][KW], vbuf[R][2][VW];
  uint16_t kscl[R][2], vscl[R][2];
  // address = chunk resource + loop-invariant lane offset + constant step offset
  struct Rsrc { __amdgpu_buffer_rsrc_t kc, ks, vc, vs; };
  // an empty range (n = 0) makes every load through it return 0 without touching memory
  auto chunk_rsrc = [&](int64_t c, int n) {
    const int64_t c0 = ts + c * CT;
    return Rsrc{make_rsrc(kc + c0 * KC, n * KC), make_rsrc(ks + c0 * KS, n * KS),
                make_rsrc(vc + c0 * VC, n * VC), make_rsrc(vs + c0 * VS, n * VS)};
  };
  auto load_k = [&](const Rsrc& r, int s) {
    const int slot = s % R;
    buf_dwords<KW>(r.kc, koff, s * STEP * KC, kbuf[slot][0]);
    buf_dwords<KW>(r.kc, koff + TPS * KC, s * STEP * KC, kbuf[slot][1]);
    if constexpr (KB == kF8) {
      kscl[slot][0] = buf_u8(r.ks, ksoff, s * STEP * KS);
      kscl[slot][1] = buf_u8(r.ks, ksoff + TPS * KS, s * STEP * KS);
    } else if constexpr (KB != 16) {
      kscl[slot][0] = buf_u16(r.ks, ksoff, s * STEP * KS);
      kscl[slot][1] = buf_u16(r.ks, ksoff + TPS * KS, s * STEP * KS);
    }
  };
  // MFMA key groups: 32 tokens each; lane (r, h) loads token r's bytes 32 b + 16 h .. + 16 of
  // every block b, and its fp16 scales (a ring of RK groups, PDK groups ahead)
  constexpr int NG = CT / 32, PDK = ONE ? NG : 2, RK = ONE ? NG : PDK + 1;
  constexpr int KQW = KB == 8 ? 4 : 2;   // code dwords per lane and block
  uint32_t kq[MQK ? RK : 1][MQK ? NB : 1][KQW];
  uint32_t kqs[MQK ? RK : 1][MQK ? (NB + 1) / 2 : 1];
  const uint32_t kqoff = (lane & 31) * KC + (KB == 8 ? 16 : 8) * (lane >> 5), kqsoff = (lane & 31) * KS;
  constexpr int KFW = MQF ? D / 8 : 1;   // fp8 code dwords per lane and group
  uint32_t kf[MQF ? RK : 1][KFW];
  uint32_t kfs[MQF ? RK : 1];
  const uint32_t kfoff = (lane & 31) * KC + (D / 2) * (lane >> 5), kfsoff = (lane & 31) * KS;
  auto load_kg = [&](const Rsrc& r, int j) {
    if constexpr (MQF) {
      const int slot = j % RK;
      buf_dwords<KFW>(r.kc, kfoff, j * 32 * KC, kf[slot]);
      if constexpr (KS == 4) kfs[slot] = __builtin_amdgcn_raw_buffer_load_b32(r.ks, (int)kfsoff, (int)(j * 32 * KS), 0);
      else kfs[slot] = buf_u16(r.ks, kfsoff, j * 32 * KS);
    }
    if constexpr (MQK) {
      const int slot = j % RK;
#pragma unroll
      for (int b = 0; b < NB; ++b) buf_dwords<KQW>(r.kc, kqoff + (KB == 8 ? 32 : 16) * b, j * 32 * KC, kq[slot][b]);
      if constexpr (NB == 4) {
        const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r.ks, (int)kqsoff, (int)(j * 32 * KS), 0);
        kqs[slot][0] = t.x;
        kqs[slot][1] = t.y;
      } else {
        static_assert(NB == 2, "head_dim 64 or 128");
        kqs[slot][0] = __builtin_amdgcn_raw_buffer_load_b32(r.ks, (int)kqsoff, (int)(j * 32 * KS), 0);
      }
    }
  };
  auto load_v = [&](const Rsrc& r, int s) {
    const int slot = s % R;
    buf_dwords<VW>(r.vc, voff, s * STEP * VC, vbuf[slot][0]);
    buf_dwords<VW>(r.vc, voff + TPS * VC, s * STEP * VC, vbuf[slot][1]);
    if constexpr (VB != 16) {
      vscl[slot][0] = buf_u16(r.vs, vsoff, s * STEP * VS);
      vscl[slot][1] = buf_u16(r.vs, vsoff + TPS * VS, s * STEP * VS);
    }
  };
  int64_t c = __builtin_amdgcn_readfirstlane(wave);
  Rsrc rc = chunk_rsrc(c, CT);
  if (c < n_chunks) {
    if constexpr (MQ) {
#pragma unroll
      for (int j = 0; j < PDK; ++j) load_kg(rc, j);
    } else {
#pragma unroll
      for (int s = 0; s < PD; ++s) load_k(rc, s);
    }
    if constexpr (ONE) {
#pragma unroll
      for (int s = 0; s < NS; ++s) load_v(rc, s);
    }
  }

  // ---- query preparation: fp32 copy, then per (head, block) two int8 digits -------
  for (int i = tid; i < GP * D; i += 256) {
    int g = i / D, e = i % D;
    s_q[g][e] = g < a.group ? load_q(a.q, a.q_dtype, (srow + g) * D + e) : 0.f;
  }
  __syncthreads();
  // one scale per query head: q ~= sq * (256 * qa + qb), |qa| <= 127, qb in [-128, 127];
  // the integer dot products then carry 16 bits of the query
  // (wave w prepares heads w, w + 4, ...: lanes split the elements, a DPP max gives amax)
  for (int g = wave; g < GP; g += 4) {
    if constexpr (KB == 16 || KB == kF8) {
      // q' = q * 2^-k with max |q'| in [2^14, 2^15): fp16 holds q' without overflow and
      // 16-bit queries exactly
      float amax = 0.f;
      for (int e = lane; e < D; e += 64) amax = fmaxf(amax, fabsf(s_q[g][e]));
      amax = wave_max(amax);
      const int sb = max((int)((__float_as_uint(amax) >> 23) & 255) - 14, 1);
      if (lane == 0) {
        s_qi[g] = __uint_as_float((uint32_t)(254 - sb) << 23);
        s_qs[g] = __uint_as_float((uint32_t)sb << 23) * a.qk_scale;
      }
    } else {
      float amax = 0.f;
      for (int e = lane; e < D; e += 64) amax = fmaxf(amax, fabsf(s_q[g][e]));
      amax = wave_max(amax);
      const float sq = amax / 32512.f;
      for (int e = lane; e < D; e += 64) {
        float v = sq > 0.f ? rintf(s_q[g][e] / sq) : 0.f;
        v = fminf(fmaxf(v, -32512.f), 32512.f);
        int Q = (int)v;
        int qa = (Q + 128) >> 8;  // floor((Q + 128) / 256)
        s_qa[g][e] = (int8_t)qa;
        s_qb[g][e] = (int8_t)(Q - 256 * qa);
      }
      if (lane == 0) s_qs[g] = sq * a.qk_scale;
    }
  }
  __syncthreads();

  uint32_t qa_r[GP][QW], qb_r[GP][QW];
  int corr_a[GP], corr_b[GP];
  float qsc[GP];        // raw score -> base-2 logit, applied once per token in phase B
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    qsc[g] = s_qs[g];
    corr_a[g] = 0;
    corr_b[g] = 0;
    if constexpr (KB == 16 || KB == kF8) {
      const float qi = s_qi[g];
#pragma unroll
      for (int j = 0; j < QW; ++j) {
        const float x0 = s_q[g][e0 + 2 * j] * qi, x1 = s_q[g][e0 + 2 * j + 1] * qi;
        const half2_t hi = pack_rne(x0, x1);
        qa_r[g][j] = __builtin_bit_cast(uint32_t, hi);
        qb_r[g][j] = __builtin_bit_cast(uint32_t, pack_rne(x0 - (float)hi.x, x1 - (float)hi.y));
      }
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

  // 8/4-bit keys on the matrix cores: v_mfma_i32_32x32x32_i8 multiplies the query's digit
  // rows (row 2 g + i = digit i of head g, zero above 2 GP) by one 32-element block of 32
  // tokens' key codes.  Lane (r, h) of a wave holds A row r = lane % 32 and B column
  // (token) r, elements 16 h .. 16 h + 15 of the block (h = lane / 32).  4-bit codes enter as
  // their nibbles u = q + 8 in the order even elements, then odd ones (k = 4 i + j is element
  // 2 j + (i & 1) + 8 (i >> 1)); the query rows follow the same order, and 8 times the
  // block's digit sums is subtracted from each result.
  // (4-bit keys at group 16 keep the VALU path: the corrections do not fit beside 16 heads'
  // accumulators)
  constexpr int NQ = (2 * GP + 7) / 8;   // quads of result rows that hold query rows
  i32x4 qA[MQK ? NB : 1];
  int qcorr[MQK && KB == 4 ? NQ : 1][2][MQK && KB == 4 ? NB : 1];   // 8 (256 S_hi + S_lo) per head, block
  if constexpr (MQK) {
    const int r = lane & 31, hl = lane >> 5;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      i32x4 x = {0, 0, 0, 0};
      if (r < 2 * GP) {
        const int8_t* src = ((r & 1) ? &s_qb[r >> 1][0] : &s_qa[r >> 1][0]) + 32 * b + 16 * hl;
        if constexpr (KB == 8) {
          x = *reinterpret_cast<const i32x4*>(src);
        } else {
          int8_t t[16];
#pragma unroll
          for (int k = 0; k < 16; ++k) t[k] = src[2 * (k & 3) + ((k >> 2) & 1) + 8 * (k >> 3)];
          __builtin_memcpy(&x, t, 16);
        }
      }
      qA[b] = x;
    }
    if constexpr (KB == 4) {
#pragma unroll
      for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int g = 4 * q + 2 * hl + h;
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            int sa = 0, sb = 0;
            if (g < GP) {
              for (int e = 0; e < kBlock; ++e) {
                sa += s_qa[g][32 * b + e];
                sb += s_qb[g][32 * b + e];
              }
            }
            qcorr[q][h][b] = 8 * (256 * sa + sb);
          }
        }
    }
  }

  // fp8 keys on the matrix cores: v_mfma_f32_32x32x16_f16 with the query rows (row g = head g,
  // or rows 2 g + i = its fp16 hi and lo parts for fp32 queries) against 32 tokens' keys
  // widened to fp16 (exactly; the block's power-of-two scale folds into the conversion).
  // Lane (r, h) loads token r's bytes [h D / 2, (h + 1) D / 2); k-step k takes its bytes
  // 8 k .. 8 k + 7 (block (h D / 2 + 8 k) / 32), and the query rows follow that order.
  constexpr int NK8 = D / 16;                       // k-steps of one 32-token group
  constexpr int QROWS = QLO ? 2 * GP : GP;
  half8_t qF[MQF ? NK8 : 1];
  if constexpr (MQF) {
    const int r = lane & 31, hl = lane >> 5;
    const int g = QLO ? r >> 1 : r;
    const bool on = r < QROWS;
    const float qi = on ? s_qi[g] : 0.f;
#pragma unroll
    for (int k = 0; k < NK8; ++k) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = on ? s_q[g][(D / 2) * hl + 8 * k + i] * qi : 0.f;
        const _Float16 hi = (_Float16)x;
        qF[k][i] = (QLO && (r & 1)) ? (_Float16)(x - (float)hi) : hi;
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

  for (; c < n_chunks; c += 4) {
    const int64_t c0 = ts + c * CT;
    const bool tail = c0 + CT > te;
    const bool more = c + 4 < n_chunks;
    const Rsrc rn = chunk_rsrc(c + 4, more ? CT : 0);
    // ---- phase A: scores ----------------------------------------------------------
    if constexpr (MQ) {
      // late iterations request the chunk's first value steps instead of key groups
      constexpr int VPER = (PD + PDK - 1) / PDK;
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        if constexpr (ONE) {
          // every code of the chunk is in flight already
        } else if (j + PDK < NG) {
          load_kg(rc, j + PDK);
        } else {
#pragma unroll
          for (int i = 0; i < VPER; ++i)
            if ((j + PDK - NG) * VPER + i < PD) load_v(rc, (j + PDK - NG) * VPER + i);
        }
        const int slot = j % RK;
        // lane (token, h) gets D rows 8 q + 4 h + {0..3}: heads 4 q + 2 h + {0, 1}, both digits
        // (or hi and lo parts); with one row per head (fp8 keys, 16-bit queries) heads 8 q + 4 h + {0..3}
        float sc[NQ][2];
#pragma unroll
        for (int q = 0; q < NQ; ++q) sc[q][0] = sc[q][1] = 0.f;
        if constexpr (MQF) {
          const int hl = lane >> 5;
          f32x16 fa = {};
#pragma unroll
          for (int k = 0; k < NK8; ++k) {
            const int blk = ((D / 2) * hl + 8 * k) / kBlock;
            const float x = __uint_as_float(((kfs[slot] >> (8 * blk)) & 255u) << 23);
            const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)kf[slot][2 * k], x, false);
            const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)kf[slot][2 * k], x, true);
            const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)kf[slot][2 * k + 1], x, false);
            const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)kf[slot][2 * k + 1], x, true);
            const half8_t kb8 = {p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
            fa = __builtin_amdgcn_mfma_f32_32x32x16_f16(qF[k], kb8, fa, 0, 0, 0);
          }
          const int t = 32 * j + (lane & 31);
          if constexpr (QLO) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
              sc[q][0] = fa[4 * q] + fa[4 * q + 1];
              sc[q][1] = fa[4 * q + 2] + fa[4 * q + 3];
            }
          } else {
#pragma unroll
            for (int q = 0; q < (GP + 7) / 8; ++q) {
              const int g0 = 8 * q + 4 * hl;
              if (g0 + 3 < GP) {
                *reinterpret_cast<float4*>(&s_sc[wave][t][g0]) =
                    make_float4(fa[4 * q], fa[4 * q + 1], fa[4 * q + 2], fa[4 * q + 3]);
              } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  if (g0 + i < GP) s_sc[wave][t][g0 + i] = fa[4 * q + i];
              }
            }
            continue;   // scores stored
          }
        }
#pragma unroll
        for (int b = 0; b < (MQK ? NB : 0); ++b) {
          i32x4 kb;
          if constexpr (KB == 8) {
            kb = i32x4{(int)kq[slot][b][0], (int)kq[slot][b][1], (int)kq[slot][b][2], (int)kq[slot][b][3]};
          } else {   // nibbles -> bytes: even elements, then odd ones
            const uint32_t w0 = kq[slot][b][0], w1 = kq[slot][b][1];
            kb = i32x4{(int)(w0 & 0x0F0F0F0Fu), (int)((w0 >> 4) & 0x0F0F0F0Fu), (int)(w1 & 0x0F0F0F0Fu),
                       (int)((w1 >> 4) & 0x0F0F0F0Fu)};
          }
          const i32x16 zero = {};
          const i32x16 dq = __builtin_amdgcn_mfma_i32_32x32x32_i8(qA[b], kb, zero, 0, 0, 0);
          const float d = h2f((uint16_t)(kqs[slot][b >> 1] >> (16 * (b & 1))));
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            int x0 = (dq[4 * q] << 8) + dq[4 * q + 1], x1 = (dq[4 * q + 2] << 8) + dq[4 * q + 3];
            if constexpr (KB == 4) {
              x0 -= qcorr[q][0][b];
              x1 -= qcorr[q][1][b];
            }
            sc[q][0] = fmaf((float)x0, d, sc[q][0]);
            sc[q][1] = fmaf((float)x1, d, sc[q][1]);
          }
        }
        const int t = 32 * j + (lane & 31);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const int g0 = 4 * q + 2 * (lane >> 5);
          if (g0 + 1 < GP) {
            *reinterpret_cast<float2*>(&s_sc[wave][t][g0]) = make_float2(sc[q][0], sc[q][1]);
          } else if (g0 < GP) {
            s_sc[wave][t][g0] = sc[q][0];
          }
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int la = s * STEP + grp, lb = la + TPS;
        if constexpr (!ONE) {
          if (s + PD < NS) load_k(rc, s + PD);
          else load_v(rc, s + PD - NS);
        }
        const uint32_t* ka = kbuf[s % R][0];
        const uint32_t* kb = kbuf[s % R][1];
        float da = 1.f, db = 1.f;
        half2_t fa[KB == kF8 ? 2 * KW : 1], fb[KB == kF8 ? 2 * KW : 1];
        if constexpr (KB == kF8) {
          // x_hat = E4M3 value * 2^(s - 127); s = 0 would be 2^-127, below every fp16
          const float xa = __uint_as_float((uint32_t)kscl[s % R][0] << 23);
          const float xb = __uint_as_float((uint32_t)kscl[s % R][1] << 23);
#pragma unroll
          for (int j = 0; j < KW; ++j) {
            fa[2 * j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)ka[j], xa, false);
            fa[2 * j + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)ka[j], xa, true);
            fb[2 * j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)kb[j], xb, false);
            fb[2 * j + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)kb[j], xb, true);
          }
        } else if constexpr (KB != 16) {
          da = h2f(kscl[s % R][0]);
          db = h2f(kscl[s % R][1]);
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
            if constexpr (QLO) {
#pragma unroll
              for (int j = 0; j < KW; ++j) {
                xa = __builtin_amdgcn_fdot2(as_h2(qb_r[g][j]), as_h2(ka[j]), xa, false);
                xb = __builtin_amdgcn_fdot2(as_h2(qb_r[g][j]), as_h2(kb[j]), xb, false);
              }
            }
            pa[g] = group_sum<LPT>(xa);
            pb[g] = group_sum<LPT>(xb);
          } else if constexpr (KB == kF8) {
            float xa = 0.f, xb = 0.f;
#pragma unroll
            for (int j = 0; j < QW; ++j) {
              xa = __builtin_amdgcn_fdot2(as_h2(qa_r[g][j]), fa[j], xa, false);
              xb = __builtin_amdgcn_fdot2(as_h2(qa_r[g][j]), fb[j], xb, false);
            }
            if constexpr (QLO) {
#pragma unroll
              for (int j = 0; j < QW; ++j) {
                xa = __builtin_amdgcn_fdot2(as_h2(qb_r[g][j]), fa[j], xa, false);
                xb = __builtin_amdgcn_fdot2(as_h2(qb_r[g][j]), fb[j], xb, false);
              }
            }
            pa[g] = group_sum<LPT>(xa);
            pb[g] = group_sum<LPT>(xb);
          } else {
            // one chain per token: high digit, times 256, then the low digit
            int ha = corr_a[g], hb = corr_a[g];
            if constexpr (KB == 8) {
              // the first product starts the chain (8-bit keys need no offset correction)
              ha = sdot4_start((int)ka[0], (int)qa_r[g][0]);
              hb = sdot4_start((int)kb[0], (int)qa_r[g][0]);
#pragma unroll
              for (int j = 1; j < KW; ++j) {
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
            // lanes of one block add their integers, then one scale per block
            ha = group_sum_i<LPB>(ha);
            hb = group_sum_i<LPB>(hb);
            float xa = (float)ha * da, xb = (float)hb * db;
            asm volatile("" : "+v"(xa), "+v"(xb));   // no multiply-add re-fusion across the DPP
            pa[g] = group_sum_rest<LPT, LPB>(xa);
            pb[g] = group_sum_rest<LPT, LPB>(xb);
          }
          // keep the last reduction step out of the store's branch (so it fuses with DPP)
          asm volatile("" : "+v"(pa[g]), "+v"(pb[g]));
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
    }
    // (the first value codes of the chunk fly during the softmax statistics)
    wave_lds_sync();
    // ---- phase B: softmax statistics, one lane per token ------------------------
    const int wr0 = lane % STEP, wr1 = (lane + 64) % STEP;
    const int wpair0 = (lane / STEP) * TPS + wr0 % TPS, whalf0 = wr0 / TPS;
    const int wpair1 = ((lane + 64) / STEP) * TPS + wr1 % TPS, whalf1 = wr1 / TPS;
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      float sa = s_sc[wave][lane][g] * qsc[g], sb = s_sc[wave][lane + 64][g] * qsc[g];
      if (tail) {  // tokens past the cached length score -inf
        if (c0 + lane >= te) sa = -INFINITY;
        if (c0 + lane + 64 >= te) sb = -INFINITY;
      }
      const float cm = wave_max(fmaxf(sa, sb));
      const float mn = fmaxf(m[g], cm);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float alpha = __builtin_amdgcn_exp2f(m[g] - mu);
      const _Float16 p0 = (_Float16)__builtin_amdgcn_exp2f(sa - mu), p1 = (_Float16)__builtin_amdgcn_exp2f(sb - mu);
      // phase C pairs token 16 s + r with 16 s + r + 8 (r < 8) in one fp16x2 word
      reinterpret_cast<_Float16*>(&s_w[wave][wpair0][g])[whalf0] = p0;
      reinterpret_cast<_Float16*>(&s_w[wave][wpair1][g])[whalf1] = p1;
      // the normalizer sums the same fp16 weights the values are weighted with
      lsum[g] = lsum[g] * alpha + ((float)p0 + (float)p1);
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
      if constexpr (ONE) {
        // one chunk per wave: nothing more to request
      } else if (s + PD < NS) load_v(rc, s + PD);
      else if constexpr (MQ) {   // the next chunk's first PDK key groups (none: an empty range)
        if (s + PD - NS < PDK) load_kg(rn, s + PD - NS);
        if (s == NS - 1) {        // chunks of fewer value steps than PDK + 1: the rest at the end
#pragma unroll
          for (int g = PD; g < PDK; ++g) load_kg(rn, g);
        }
      } else {
        load_k(rn, s + PD - NS);   // the next chunk (none: an empty range, no traffic)
      }
      const uint32_t* va = vbuf[s % R][0];
      const uint32_t* vb = vbuf[s % R][1];
      // weights of the token pair: fp16 p times the tokens' value scales (packed fp16)
      half2_t w[GP];
      const uint32_t* wp = &s_w[wave][s * TPS + grp][0];
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        w[g] = as_h2(wp[g]);
        if constexpr (VB != 16) w[g] = w[g] * as_h2((uint32_t)vscl[s % R][0] | ((uint32_t)vscl[s % R][1] << 16));
        wsum[g] = __builtin_amdgcn_fdot2(w[g], as_h2(0x3C003C00u), wsum[g], false);
      }
#pragma unroll
      for (int j = 0; j < VW; ++j) {
        if constexpr (VB == 4) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t sel = (uint32_t)k | (0x0cu << 8) | ((uint32_t)(4 + k) << 16) | (0x0cu << 24);
            // the whole byte (even nibble + 16 x odd nibble) and the odd nibble alone; the
            // epilogue takes the even sum as their difference (no mask for the even nibble)
            const uint32_t pr = __builtin_amdgcn_perm(vb[j], va[j], sel);
            const half2_t by = as_h2(pr), od = as_h2(pr & 0x00F000F0u);
#pragma unroll
            for (int g = 0; g < GP; ++g) {
              acc[g][8 * j + 2 * k] = __builtin_amdgcn_fdot2(w[g], by, acc[g][8 * j + 2 * k], false);
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
    rc = rn;
  }

  // ---- epilogue: wave partials -> workgroup partial -------------------------------
  // the lane's sums of its elements e0 .. e0 + E - 1, then one reduce-scatter over the lanes
  // that share those elements (lane % LPT): each lane ends with GP * D / 64 of the wave's sums
  constexpr int NV = GP * E, NF = GP * D / 64;
  float ov[NV];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float o;
      if constexpr (VB == 4)
        o = ((e & 1) ? acc[g][e] * 1048576.f : (acc[g][e] - acc[g][e + 1]) * 16777216.f) - 8.f * wsum[g];
      else if constexpr (VB == 8) o = acc[g][e] * 16777216.f - 128.f * wsum[g];
      else o = acc[g][e];
      ov[g * E + e] = o;
    }
  }
  reduce_scatter<LPT>(ov, lane);
  {
    const int first = reduce_scatter_first<LPT, NV>(lane);
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int idx = first + i, g = idx / E;
      s_o[wave][g][e0 + idx % E] = ov[i];
    }
  }
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    const float lw = wave_sum(lsum[g]);
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
    if (!part) {
      a.out[row * D + e] = o / l;
    } else {
      float* p = a.ws + (row * a.n_splits + split) * (D + 2);
      st_partial(p + e, o);
      if (e == 0) {
        st_partial(p + D, M);
        st_partial(p + D + 1, l);
      }
    }
  }
  if (part && a.fused) merge_if_last<D>(a, S, n_merge, srow, vhead, tid, &s_last);
  if constexpr (STREAM) __syncthreads();   // the next session's query preparation rewrites LDS
  } while (STREAM && blk < blk_end);
}

template <int GP>
constexpr int lane_elems() { return GP <= 2 ? 32 : (GP == 4 ? 16 : 8); }

// The single-chunk variant keeps a whole chunk's key and value codes in registers: only where
// they take at most 64 registers a lane (and the query group is small) does it fit beside the
// rest of the kernel.
template <int KB, int VB, int D, int GP>
constexpr bool one_chunk_variant() {
  constexpr int kbytes = KB == 16 ? 2 * D : (KB == 4 ? D / 2 : D), vbytes = VB == 16 ? 2 * D : (VB == 4 ? D / 2 : D);
  return GP <= 8 && kDecodeChunk * (kbytes + vbytes) / 64 <= 256;
}

template <int KB, int VB, int D, int GP>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
  constexpr int E = lane_elems<GP>();
  constexpr bool HL = KB == kF8 || KB == 16;   // keys met by an fp16 query: fp32 queries add a low part
  if (a.stream) {
    const dim3 grid(a.hkv * a.hsplit, a.n_wg, 1);
    if (HL && a.q_dtype == 0) hipLaunchKernelGGL((decode_kernel<KB, VB, D, GP, E, HL, false, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((decode_kernel<KB, VB, D, GP, E, false, false, true>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const dim3 grid(a.hkv * a.hsplit, a.compact ? a.n_pieces : a.n_sess, a.compact ? 1 : a.n_splits);
  const bool one = one_chunk_variant<KB, VB, D, GP>() && a.one_chunk;
  constexpr bool OK1 = one_chunk_variant<KB, VB, D, GP>();
  if (HL && a.q_dtype == 0) {
    if (one) hipLaunchKernelGGL((decode_kernel<KB, VB, D, GP, E, HL, OK1>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((decode_kernel<KB, VB, D, GP, E, HL>), grid, dim3(256), 0, s, a);
  } else {
    if (one) hipLaunchKernelGGL((decode_kernel<KB, VB, D, GP, E, false, OK1>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((decode_kernel<KB, VB, D, GP, E>), grid, dim3(256), 0, s, a);
  }
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

template <int KB, int VB, int D, bool ST, bool QL>
const void* ptr_g(int gp) {
  switch (gp) {
    case 1: return reinterpret_cast<const void*>(&decode_kernel<KB, VB, D, 1, lane_elems<1>(), QL, false, ST>);
    case 2: return reinterpret_cast<const void*>(&decode_kernel<KB, VB, D, 2, lane_elems<2>(), QL, false, ST>);
    case 4: return reinterpret_cast<const void*>(&decode_kernel<KB, VB, D, 4, lane_elems<4>(), QL, false, ST>);
    case 8: return reinterpret_cast<const void*>(&decode_kernel<KB, VB, D, 8, lane_elems<8>(), QL, false, ST>);
    default: return reinterpret_cast<const void*>(&decode_kernel<KB, VB, D, 16, lane_elems<16>(), QL, false, ST>);
  }
}

template <int KB, int VB, bool QL = false>
const void* ptr_d(int d, int gp, bool st) {
  if (st) return d == 64 ? ptr_g<KB, VB, 64, true, QL>(gp) : ptr_g<KB, VB, 128, true, QL>(gp);
  return d == 64 ? ptr_g<KB, VB, 64, false, false>(gp) : ptr_g<KB, VB, 128, false, false>(gp);
}

}  // namespace

const void* decode_kernel_for(int kbits, int vbits, int d, int gp, bool stream, bool q_fp32) {
  if (kbits == 16) return q_fp32 && stream ? ptr_d<16, 16, true>(d, gp, true) : ptr_d<16, 16>(d, gp, stream);
  if (kbits == kF8) return q_fp32 && stream ? ptr_d<kF8, 4, true>(d, gp, true) : ptr_d<kF8, 4>(d, gp, stream);
  if (kbits == 8 && vbits == 8) return ptr_d<8, 8>(d, gp, stream);
  if (kbits == 8) return ptr_d<8, 4>(d, gp, stream);
  if (vbits == 8) return ptr_d<4, 8>(d, gp, stream);
  return ptr_d<4, 4>(d, gp, stream);
}

hipError_t launch_decode(const DecodeArgs& a, int kbits, int vbits, int d, int gp, hipStream_t s) {
  if (kbits == 16 && vbits == 16) return launch_d<16, 16>(a, d, gp, s);
  if (kbits == 8 && vbits == 8) return launch_d<8, 8>(a, d, gp, s);
  if (kbits == 8 && vbits == 4) return launch_d<8, 4>(a, d, gp, s);
  if (kbits == 4 && vbits == 8) return launch_d<4, 8>(a, d, gp, s);
  if (kbits == 4 && vbits == 4) return launch_d<4, 4>(a, d, gp, s);
  if (kbits == kF8 && vbits == 4) return launch_d<kF8, 4>(a, d, gp, s);
  return hipErrorInvalidValue;
}

}  // namespace kvq

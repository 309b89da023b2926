// One output row of the split merge (second pass of split attention): per-split partials
// (o unnormalized, m = running max in log2 units, l = sum of 2^(s - m)) become
//   M = max_s m_s,  out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,
// splits with m = -inf weighing nothing.  The standalone merge kernels and the decode
// kernel's own last-workgroup merge both call these, so a fused call and the two passes
// run separately under the same plan give the same bits.
#pragma once

#include "wave_ops.h"

namespace kvq {

// A partial read back in the launch that wrote it (the decode kernel's own merge) is loaded
// with an agent-scope atomic load, which reads past a stale line of this XCD's L2; the
// standalone merge kernels, launched after the writer, load plainly.  The values are the same.
template <bool COHERENT>
__device__ __forceinline__ float ld_partial(const float* p) {
  if constexpr (COHERENT) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}

// Few splits of head_dim 64 or 128 take the sequential form, more the lane-per-split form.
constexpr int kRowsKernelSplits = 4;
__host__ __device__ constexpr bool merge_seq_form(int d, int n_splits) {
  return (d == 64 || d == 128) && n_splits <= kRowsKernelSplits;
}

// Lane-per-split form, one whole wave per row (lane = this lane's index, every lane
// active): lane s loads split s's (m, l) together, so the statistics of 64 splits take one
// round trip; the weights 2^(m_s - M) / L go to every lane through readlane, and each lane
// sums the splits for its elements of head_dim, 16 splits' loads in flight at a time.
// p: the row's ns >= 1 splits of d + 2 floats.  Loads past the row's splits or head_dim read
// the last split or element instead (addresses clamped, values then dropped), so every batch
// goes out unconditionally.
template <bool COHERENT = false>
__device__ inline void merge_row_wave(const float* p, int ns, int d, float* out, int lane) {
  const int stride = d + 2, sl = ns - 1, el = min(lane, d - 1);
  // the first 16 splits' element `lane` go out with the statistics (at head_dim 64 and up to
  // 16 splits, the whole row in one round trip)
  float x0[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float v = ld_partial<COHERENT>(p + min(i, sl) * stride + el);
    x0[i] = lane < d && i < ns ? v : 0.f;
  }
  float m0, l0;   // split `lane`'s statistics, of the first 64 splits
  {
    const float mv = ld_partial<COHERENT>(p + min(lane, sl) * stride + d);
    const float lv = ld_partial<COHERENT>(p + min(lane, sl) * stride + d + 1);
    m0 = lane < ns ? mv : -INFINITY;
    l0 = lane < ns ? lv : 0.f;
  }
  float M = wave_max(m0);
  for (int s0 = 64; s0 < ns; s0 += 64) {
    const float mv = ld_partial<COHERENT>(p + min(s0 + lane, sl) * stride + d);
    M = fmaxf(M, wave_max(s0 + lane < ns ? mv : -INFINITY));
  }
  float L = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    const int s = s0 + lane;
    float ms = m0, ls = l0;
    if (s0 > 0) {
      const float mv = ld_partial<COHERENT>(p + min(s, sl) * stride + d);
      const float lv = ld_partial<COHERENT>(p + min(s, sl) * stride + d + 1);
      ms = s < ns ? mv : -INFINITY;
      ls = s < ns ? lv : 0.f;
    }
    L += wave_sum(ms != -INFINITY ? __builtin_amdgcn_exp2f(ms - M) * ls : 0.f);
  }
  const float inv = 1.f / L;
  for (int e0 = 0; e0 < d; e0 += 64) {
    const int e = e0 + lane, ec = min(e, d - 1);
    const bool on = e < d;
    float o = 0.f;
    for (int s0 = 0; s0 < ns; s0 += 64) {
      const int s = s0 + lane;
      // this lane's split weight, handed to every lane below
      float ms = m0;
      if (s0 > 0) {
        const float mv = ld_partial<COHERENT>(p + min(s, sl) * stride + d);
        ms = s < ns ? mv : -INFINITY;
      }
      const float w = ms != -INFINITY ? __builtin_amdgcn_exp2f(ms - M) * inv : 0.f;
      const int n = min(64, ns - s0);
      for (int j = 0; j < n; j += 16) {
        float x[16];
        if (e0 == 0 && s0 == 0 && j == 0) {   // wave-uniform: the batch loaded up front
#pragma unroll
          for (int i = 0; i < 16; ++i) x[i] = x0[i];
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float v = ld_partial<COHERENT>(p + (s0 + min(j + i, n - 1)) * stride + ec);
            x[i] = on && j + i < n ? v : 0.f;
          }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) o = fmaf(readlane(w, min(j + i, 63)), x[i], o);
      }
    }
    if (on) out[e] = o;
  }
}

// Sequential form, D = 64 or 128 and 1 <= ns <= kRowsKernelSplits: lane sub of the row's D / 8
// lanes writes elements 8 sub .. 8 sub + 7.  Each lane loads every split's (m, l) and its
// own elements of every split in one round trip, so no cross-lane reduction sits between the
// statistics and the weighted sum; the normalizer is summed in split order.
template <int D, bool COHERENT = false>
__device__ inline void merge_row_seq(const float* p, int ns, int sub, float* out) {
  constexpr int STRIDE = D + 2, NS = kRowsKernelSplits;
  float m[NS], l[NS], x[NS][8];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    m[s] = -INFINITY;
    l[s] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) x[s][i] = 0.f;
    // splits past ns read split ns - 1 (a clamped address; the values are dropped), so the
    // loads of every split go out together
    const int sc = min(s, ns - 1);
    const float mv = ld_partial<COHERENT>(p + sc * STRIDE + D), lv = ld_partial<COHERENT>(p + sc * STRIDE + D + 1);
    const float* xs = p + sc * STRIDE + 8 * sub;
    float xv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float2 v;
      if constexpr (COHERENT) {
        v.x = ld_partial<true>(xs + 2 * i);
        v.y = ld_partial<true>(xs + 2 * i + 1);
      } else {
        v = reinterpret_cast<const float2*>(xs)[i];   // 8-byte aligned rows
      }
      xv[2 * i] = v.x;
      xv[2 * i + 1] = v.y;
    }
    if (s < ns) {
      m[s] = mv;
      l[s] = lv;
#pragma unroll
      for (int i = 0; i < 8; ++i) x[s][i] = xv[i];
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < NS; ++s) M = fmaxf(M, m[s]);
  float L = 0.f;
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (m[s] != -INFINITY) L += __builtin_amdgcn_exp2f(m[s] - M) * l[s];
  const float inv = 1.f / L;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s >= ns) break;
    const float w = m[s] != -INFINITY ? __builtin_amdgcn_exp2f(m[s] - M) * inv : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = fmaf(w, x[s][i], o[i]);
  }
  float4* dst = reinterpret_cast<float4*>(out + 8 * sub);
  dst[0] = make_float4(o[0], o[1], o[2], o[3]);
  dst[1] = make_float4(o[4], o[5], o[6], o[7]);
}

}  // namespace kvq

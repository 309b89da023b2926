// Second pass of split attention: combine per-split partials (o unnormalized,
// m = running max in log2 units, l = sum of 2^(s - m)) into the normalized output,
//   M = max_s m_s,  o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// One wave per output row.  Lane s loads split s's (m, l), so the statistics of up to 64
// splits take one round trip; the weights w_s = 2^(m_s - M) / L then go to every lane
// through readlane, and each lane sums the splits for its elements of head_dim.  Splits
// that saw no token carry m = -inf, l = 0 and weigh nothing; a decode batch launched with
// its busy workgroups only names, per session, how many leading splits to read.
#include "kvq_internal.h"
#include "wave_ops.h"

namespace kvq {
namespace {

__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;   // wave-uniform
  const int stride = a.d + 2;
  const float* p = a.ws + row * a.n_splits * stride;
  const int ns = a.rows_per_sess > 0 ? a.n_valid[row / a.rows_per_sess] : a.n_splits;   // splits to read
  // statistics, 64 splits at a time
  float M = -INFINITY;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    const float ms = s0 + lane < ns ? p[(s0 + lane) * stride + a.d] : -INFINITY;
    M = fmaxf(M, wave_max(ms));
  }
  float L = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    const int s = s0 + lane;
    float w = 0.f;
    if (s < ns) {
      const float ms = p[s * stride + a.d];
      if (ms != -INFINITY) w = __builtin_amdgcn_exp2f(ms - M) * p[s * stride + a.d + 1];
    }
    L += wave_sum(w);
  }
  const float inv = 1.f / L;
  for (int e0 = 0; e0 < a.d; e0 += 64) {
    const int e = e0 + lane;
    const bool on = e < a.d;
    float o = 0.f;
    for (int s0 = 0; s0 < ns; s0 += 64) {
      const int s = s0 + lane;
      float w = 0.f;   // this lane's split weight, handed to every lane below
      if (s < ns) {
        const float ms = p[s * stride + a.d];
        if (ms != -INFINITY) w = __builtin_amdgcn_exp2f(ms - M) * inv;
      }
      const int n = min(64, ns - s0);
      // four splits' loads are issued before their products are summed
      for (int j = 0; j < n; j += 4) {
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = on && j + i < n ? p[(s0 + j + i) * stride + e] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) o = fmaf(readlane(w, min(j + i, 63)), x[i], o);
      }
    }
    if (on) a.out[row * a.d + e] = o;
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  const int64_t blocks = (a.rows + 3) / 4;
  if (blocks <= 0 || blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq

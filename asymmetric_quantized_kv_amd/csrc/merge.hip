// Second pass of split attention: combine per-split partials (o unnormalized,
// m = running max in log2 units, l = sum of 2^(s - m)) into the normalized output,
//   M = max_s m_s,  o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// One wave per output row; lanes stride over head_dim.  Splits that saw no token
// carry m = -inf and l = 0 and drop out.
#include "kvq_internal.h"

namespace kvq {
namespace {

__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int stride = a.d + 2;
  const float* p = a.ws + row * a.n_splits * stride;
  float M = -INFINITY;
  for (int s = 0; s < a.n_splits; ++s) M = fmaxf(M, p[s * stride + a.d]);
  float l = 0.f;
  for (int s = 0; s < a.n_splits; ++s) {
    const float ms = p[s * stride + a.d];
    if (ms != -INFINITY) l += __builtin_amdgcn_exp2f(ms - M) * p[s * stride + a.d + 1];
  }
  const float inv = 1.f / l;
  for (int e = lane; e < a.d; e += 64) {
    float o = 0.f;
    for (int s = 0; s < a.n_splits; ++s) {
      const float ms = p[s * stride + a.d];
      if (ms != -INFINITY) o += __builtin_amdgcn_exp2f(ms - M) * p[s * stride + e];
    }
    a.out[row * a.d + e] = o * inv;
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

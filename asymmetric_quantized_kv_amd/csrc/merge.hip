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

// Few splits (at most kRowsKernelSplits) and head_dim D = 8 LPR (64 and 128): LPR lanes per
// row, eight elements each, 256 / LPR rows per workgroup.  Each lane reads every split's
// (m, l) itself (the row's lanes read the same words), so no cross-lane reduction sits
// between the statistics and the weighted sum, and a row's loads are issued back to back.
// Same sums as above, the normalizer in split order.  (With many splits the lane-per-split
// kernel above wins: here every lane walks the splits one after the other.)
template <int LPR>
__global__ __launch_bounds__(256) void merge_rows_kernel(MergeArgs a) {
  constexpr int D = 8 * LPR, STRIDE = D + 2;
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR;
  const int sub = threadIdx.x % LPR;
  if (row >= a.rows) return;
  const float* p = a.ws + row * a.n_splits * STRIDE;
  const int ns = a.rows_per_sess > 0 ? a.n_valid[row / a.rows_per_sess] : a.n_splits;   // splits to read
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, p[s * STRIDE + D]);
  float L = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float ms = p[s * STRIDE + D];
    if (ms != -INFINITY) L += __builtin_amdgcn_exp2f(ms - M) * p[s * STRIDE + D + 1];
  }
  const float inv = 1.f / L;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < ns; ++s) {
    const float ms = p[s * STRIDE + D];
    const float w = ms != -INFINITY ? __builtin_amdgcn_exp2f(ms - M) * inv : 0.f;
    const float2* x = reinterpret_cast<const float2*>(p + s * STRIDE + 8 * sub);   // 8-byte aligned rows
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float2 v = x[i];
      o[2 * i] = fmaf(w, v.x, o[2 * i]);
      o[2 * i + 1] = fmaf(w, v.y, o[2 * i + 1]);
    }
  }
  float4* dst = reinterpret_cast<float4*>(a.out + row * D + 8 * sub);
  dst[0] = make_float4(o[0], o[1], o[2], o[3]);
  dst[1] = make_float4(o[4], o[5], o[6], o[7]);
}

}  // namespace

constexpr int kRowsKernelSplits = 4;

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  if ((a.d == 64 || a.d == 128) && a.n_splits <= kRowsKernelSplits) {
    const int lpr = a.d / 8;
    const int64_t blocks = (a.rows * lpr + 255) / 256;
    if (blocks <= 0 || blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (lpr == 8)
      hipLaunchKernelGGL(merge_rows_kernel<8>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(merge_rows_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const int64_t blocks = (a.rows + 3) / 4;
  if (blocks <= 0 || blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq

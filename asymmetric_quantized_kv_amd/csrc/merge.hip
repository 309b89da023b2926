// Second pass of split attention: combine per-split partials (o unnormalized,
// m = running max in log2 units, l = sum of 2^(s - m)) into the normalized output,
//   M = max_s m_s,  o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// One wave per output row.  Lane s loads split s's (m, l), so the statistics of up to 64
// splits take one round trip; the weights w_s = 2^(m_s - M) / L then go to every lane
// through readlane, and each lane sums the splits for its elements of head_dim.  Splits
// that saw no token carry m = -inf, l = 0 and weigh nothing; a decode batch launched with
// its busy workgroups only names, per session, how many leading splits to read.
#include "kvq_internal.h"
#include "merge_row.h"

namespace kvq {
namespace {

__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;   // wave-uniform
  const int ns = a.rows_per_sess > 0 ? a.n_valid[row / a.rows_per_sess] : a.n_splits;   // splits to read
  merge_row_wave(a.ws + row * a.n_splits * (a.d + 2), ns, a.d, a.out + row * a.d, threadIdx.x & 63);
}

// Few splits: LPR = D / 8 lanes per row, 256 / LPR rows per workgroup.  (With many splits
// the lane-per-split kernel above wins: here every lane walks the splits one after the other.)
template <int LPR>
__global__ __launch_bounds__(256) void merge_rows_kernel(MergeArgs a) {
  constexpr int D = 8 * LPR;
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR;
  if (row >= a.rows) return;
  const int ns = a.rows_per_sess > 0 ? a.n_valid[row / a.rows_per_sess] : a.n_splits;   // splits to read
  merge_row_seq<D>(a.ws + row * a.n_splits * (D + 2), ns, threadIdx.x % LPR, a.out + row * D);
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  if (merge_seq_form(a.d, a.n_splits)) {
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

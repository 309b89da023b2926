// Library-owned device scratch for the allocation-free decode entry point
// (kv_attend_decode_static): the split partials of a decode call live in a file-scope
// device array instead of a caller workspace, so the call needs no allocation at all.
//
// The array's name is a host-side stand-in in host code: its device address is looked up
// once per device with hipGetSymbolAddress (with that device current) and kept; only that
// address is ever handed to kernels.  Every device holds its own copy of the array, from
// module load until the process ends.  All calls on one device share it, so calls that
// overlap on one device race for it.
#include "kvq_internal.h"

#include <mutex>

namespace kvq {
namespace {

__device__ __align__(256) float scratch[kStaticScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices];

}  // namespace

hipError_t static_scratch(int device, float** ptr) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != device) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = static_cast<float*>(p);
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace kvq

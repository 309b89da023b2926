// Stand-ins for the kernel side of libkvq (the launchers and kernel symbols the host code
// links against), so that the host code alone can be built with host sanitizers.  Every
// launch fails; the host checks the sanitized build exercises run before any launch.
#include "kvq_internal.h"

namespace kvq {
hipError_t launch_append(const AppendArgs&, int, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_decode(const DecodeArgs&, int, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_chunk(const ChunkArgs&, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_merge(const MergeArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t static_scratch(int, float** ptr) {
  *ptr = nullptr;
  return hipErrorInvalidValue;
}
const void* decode_kernel_for(int, int, int, int, bool, bool) { return nullptr; }
const void* chunk_kernel_for(int, int, int, bool) { return nullptr; }
}  // namespace kvq

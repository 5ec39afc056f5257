// Small utility kernels.  Counters are cleared with a kernel rather than hipMemsetAsync so
// that callers may capture the whole step in a HIP graph.
#include "device_common.hpp"
#include "elb_kernels.h"

namespace elb {
namespace {

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t value) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = value;
}

// Does nothing: a time stamp in the stream.  The next kernel starts as it ends, with no barrier
// packet between them (an event record puts one there and delays the next dispatch).
__global__ __launch_bounds__(64) void mark_kernel() {}

}  // namespace

hipError_t launch_mark(hipEvent_t ev, hipStream_t stream) {
  return launch_timed(mark_kernel, dim3(1), dim3(64), 0, stream, nullptr, ev);
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t value, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  return launch(fill_i32_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, stream, p, n, value);
}

}  // namespace elb

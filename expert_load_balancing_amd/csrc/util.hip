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

// out[0] ^= the XOR of every 32-bit word of src[0 .. n16): a plain streaming read of HBM, the
// measured counterpart of the published read bandwidth.  Each workgroup reads one contiguous
// range, its threads 16 bytes apart, eight non-temporal 16-byte loads in flight per thread; one
// atomic per wave.  512 workgroups (two per CU) of contiguous ranges streamed 7.1 TB/s on the
// MI355X, against 5.9 TB/s for a grid-strided walk of the same loads.
constexpr int kStreamBlocks = 512;
constexpr int kStreamUnroll = 8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void stream_xor_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                         uint32_t* __restrict__ out) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per;
  const int64_t hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  int64_t i = lo + threadIdx.x;
  for (; i + (kStreamUnroll - 1) * 256 < hi; i += kStreamUnroll * 256) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < hi; i += 256) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
  if ((threadIdx.x & 63) == 0) atomicXor(out, acc);
}

}  // namespace

hipError_t launch_stream_xor(const void* src, int64_t n16, uint32_t* out, hipStream_t stream) {
  if (n16 <= 0) return hipSuccess;
  const int64_t blocks = (n16 + 256 * kStreamUnroll - 1) / (256 * kStreamUnroll);
  return launch(stream_xor_kernel, dim3((unsigned)(blocks < kStreamBlocks ? blocks : kStreamBlocks)), dim3(256), 0,
                stream, static_cast<const u32x4*>(src), n16, out);
}

hipError_t launch_mark(hipEvent_t ev, hipStream_t stream) {
  return launch_timed(mark_kernel, dim3(1), dim3(64), 0, stream, nullptr, ev);
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t value, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  return launch(fill_i32_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, stream, p, n, value);
}

}  // namespace elb

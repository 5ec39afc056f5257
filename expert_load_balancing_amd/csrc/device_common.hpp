// Small device helpers shared by the HIP kernels of this library.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace elb {

// Workgroup barrier that orders LDS traffic only.  A plain __syncthreads() also waits for
// every global load still in flight (s_waitcnt vmcnt(0)), which would drain the software
// prefetch of the next tile; fencing the "local" address space alone keeps it in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Orders this wave's own LDS writes before its later LDS reads of other lanes' data.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

}  // namespace elb

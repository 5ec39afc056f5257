// Internal interface between the C-ABI layer (elb_api.cpp) and the HIP kernels.
// Not installed; the public interface is include/elb.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <tuple>
#include <utility>

namespace elb {

struct RouterArgs {
  const void* x;
  int dtype;  // ELB_F32 / ELB_BF16
  int64_t T;
  int d;
  const void* w;
  const float* bias;
  int n_experts;
  int k;
  uint32_t flags;
  int32_t* idx;
  float* gates;
  int32_t* counts;
  float* logits;
  float* lse;
};

// Launch `kernel` and return the runtime's verdict instead of dropping it.
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t stream,
                  Args&&... args) {
  std::tuple<KArgs...> held(std::forward<Args>(args)...);
  void* ptrs[sizeof...(KArgs)];
  std::apply([&](auto&... a) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&a)), ...);
  }, held);
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, shmem, stream);
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t value, hipStream_t stream);

bool router_mfma_applies(const RouterArgs& a);
hipError_t launch_router_mfma(const RouterArgs& a, hipStream_t stream);
hipError_t launch_router_generic(const RouterArgs& a, hipStream_t stream);

int64_t dispatch_tile_entries(int64_t total);
size_t dispatch_workspace_bytes(int64_t total, int n_experts);
hipError_t launch_dispatch(const int32_t* idx, int64_t total, int n_experts, void* workspace,
                           int32_t* offsets, int32_t* perm, int32_t* inv, hipStream_t stream);

// mode < 0: MaxVio only (no update).
hipError_t launch_balance(const int32_t* counts, int n_experts, int mode, float lambda, float beta,
                          float kappa, float gamma, float* bias, float* momentum, float* delta_b,
                          float* maxvio, hipStream_t stream);

}  // namespace elb

// Internal interface between the C-ABI layer (elb_api.cpp) and the HIP kernels.
// Not installed; the public interface is include/elb.h.
#pragma once

#include <hip/hip_ext.h>
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
  int32_t* tile_loads;   // NULL, or the dispatch workspace's [n_experts][loads_stride] table:
  int64_t loads_stride;  // the MFMA kernel then stores each 256-token tile's loads in it
  hipEvent_t ev_stop = nullptr;  // NULL, or an event that takes the router kernel's end time stamp
};

// One bias update / MaxVio (balance_wave.hpp).  mode < 0: MaxVio only.
struct BalanceArgs {
  int32_t* counts;
  int n;
  int mode;
  float lambda, beta, kappa, gamma;
  int clear;  // zero `counts` once read
  float* bias;
  float* momentum;
  float* delta_b;
  float* maxvio;
};

// Launch `kernel` and return the runtime's launch status instead of dropping it.  With an event
// created with hipEventDisableSystemFence as ev_stop, the dispatch itself stamps its end time
// into it (hipExtLaunchKernel); ev_start is recorded as a marker just before the dispatch.
template <typename... KArgs, typename... Args>
hipError_t launch_timed(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t stream,
                        hipEvent_t ev_start, hipEvent_t ev_stop, Args&&... args) {
  std::tuple<KArgs...> held(std::forward<Args>(args)...);
  void* ptrs[sizeof...(KArgs)];
  std::apply([&](auto&... a) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&a)), ...);
  }, held);
  if (ev_start == nullptr && ev_stop == nullptr)
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, shmem, stream);
  return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, shmem, stream, ev_start,
                            ev_stop, 0);
}
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t stream,
                  Args&&... args) {
  return launch_timed(kernel, grid, block, shmem, stream, nullptr, nullptr, std::forward<Args>(args)...);
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t value, hipStream_t stream);
// out[0] ^= XOR of the n16 16-byte words at src (a streaming read; src 16-byte aligned).
hipError_t launch_stream_xor(const void* src, int64_t n16, uint32_t* out, hipStream_t stream);
// An empty one-wave kernel whose end time stamp goes into `ev`.
hipError_t launch_mark(hipEvent_t ev, hipStream_t stream);

bool router_mfma_applies(const RouterArgs& a);
// true: the MFMA router runs 256-token tiles for T tokens and fills the dispatch's loads table;
// false: 128-token tiles (batches of at most 128 tokens per CU; 64-token tiles for at most 64
// per CU), and the dispatch counts itself.
bool router_mfma_full_tile(int64_t T);
hipError_t launch_router_mfma(const RouterArgs& a, hipStream_t stream);
hipError_t launch_router_generic(const RouterArgs& a, hipStream_t stream);

// Dispatch works on tiles of kDispatchTile tokens (all K slots of each): the MFMA router's own
// tile, so that kernel can hand over its per-tile loads.
constexpr int kDispatchTile = 256;
struct DispatchGeom {
  int64_t n_tiles;  // ceil(T / kDispatchTile)
  int64_t stride;   // row stride of the loads table: n_tiles rounded up to a multiple of 4
};
DispatchGeom dispatch_geometry(int64_t T);
size_t dispatch_workspace_bytes(int64_t T, int n_experts);
// The static dispatch workspace of elb_router_dispatch_noalloc (dispatch.hip): its size, and its
// device address on the device of `stream` (looked up once per device).
constexpr size_t kDispatchScratchBytes = size_t(8) << 20;
hipError_t dispatch_scratch(hipStream_t stream, void** ptr);
// loads_ready: the router kernel already filled the loads table for this batch.
// counts: NULL, or the expert loads that the scan sets to (accumulate: adds) this batch's totals.
// update: NULL, or a bias update to run beside the scatter (one extra workgroup).
// ev_stop: NULL, or an event that takes the end time stamp of the dispatch's last kernel.
hipError_t launch_dispatch(const int32_t* idx, int64_t T, int k, int n_experts, void* workspace, bool loads_ready,
                           int32_t* counts, bool accumulate, const BalanceArgs* update, int32_t* offsets,
                           int32_t* perm, int32_t* inv,
                           hipStream_t stream, hipEvent_t ev_stop = nullptr);

// ev_stop (optional): an event that takes the kernel's end time stamp.
hipError_t launch_balance(const BalanceArgs& a, hipStream_t stream, hipEvent_t ev_stop = nullptr);
// n_layers independent updates, layer l at offset l * a.n (maxvio at 2 l).
hipError_t launch_balance_layers(const BalanceArgs& a, int n_layers, hipStream_t stream,
                                 hipEvent_t ev_stop = nullptr);
hipError_t launch_zloss(const float* lse, int64_t T, float* out, hipStream_t stream, hipEvent_t ev_stop = nullptr);

// router_backward.hip (bf16, d % 64 == 0).
struct BackwardArgs {
  const void* x;
  int64_t T;
  int d;
  const void* w;
  int n_experts;
  int k;
  int normalize;
  const int32_t* idx;
  const float* dgates;
  float zloss_coef;
  void* dx;      // [T][d] fp32 (bf16 with dx_bf16), or NULL
  bool dx_bf16;
  float* dw;     // [n_experts][d] fp32, or NULL
};
struct BackwardPlan {
  int64_t Q;        // 64-token stages of the batch
  int n_col;        // 256-column tiles of d
  int splits;       // token ranges of dW (one fp32 partial each)
  uint16_t* dz;     // dL/dz, token-major [T][256] bf16
  float* part;      // dW partials [splits][256][d] fp32
  size_t bytes;     // workspace bytes
};
BackwardPlan backward_plan(int64_t T, int d, void* workspace);  // workspace may be NULL (sizes only)
hipError_t launch_router_backward(const BackwardArgs& a, const BackwardPlan& p, hipStream_t stream);

// moe_ops.hip: row_bytes % 16 == 0; x, xp, eo, y 16-byte aligned.
hipError_t launch_permute_rows(const void* x, int64_t T, int64_t row_bytes, int k, const int32_t* inv, void* xp,
                               hipStream_t stream);
hipError_t launch_combine(const void* eo, int in_dtype, int64_t T, int d, int k, const int32_t* inv,
                          const float* gates, void* y, int out_dtype, hipStream_t stream);

}  // namespace elb

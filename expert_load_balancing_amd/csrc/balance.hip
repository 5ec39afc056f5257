// Expert-bias update / MaxVio launches (the arithmetic and its citations live in
// balance_wave.hpp, which the dispatch scatter also runs as an extra workgroup when a routed
// step asks for the update), and the router z-loss reduction.
#include "balance_wave.hpp"

namespace elb {
namespace {

// One workgroup (one wave) per MoE layer; layer l's rows of counts, b, m, delta_b are
// [l * n, (l + 1) * n) and its MaxVio pair is maxvio[2 l], maxvio[2 l + 1].  Layers share
// nothing: each has its own loads, bias and momentum ("SMEBU Load Balancing", "How it works":
// the update is stated per router).
__global__ __launch_bounds__(64) void balance_layers_kernel(BalanceArgs a) {
  const int64_t off = (int64_t)blockIdx.x * a.n;
  BalanceArgs l = a;
  l.counts += off;
  if (l.bias != nullptr) l.bias += off;
  if (l.momentum != nullptr) l.momentum += off;
  if (l.delta_b != nullptr) l.delta_b += off;
  if (l.maxvio != nullptr) l.maxvio += 2 * (int64_t)blockIdx.x;
  balance_wave(l);
}

// Router z-loss from per-token log-sum-exps: mean_t lse_t^2 (talk summary "Arcee Halts 400B
// Blackwell Model Collapse With Dynamic Router Biases", section "Precision Fallbacks, Loss
// Stabilization, and MaxVio as Data Telemetry": L_z = log^2 sum e^x).  One workgroup; each
// thread adds its share in float64 in a fixed order, then a reduction per wave and the waves in
// order: the same bits every run.  The share: the elements before the first 16-byte boundary
// (at most 3) and after the last one go to thread 0; the 4-element chunks between them go to the
// threads in turn (chunk c to thread c % 1024), each thread keeping eight 16-byte loads in flight
// (128 KiB over the workgroup) and adding their elements in index order.
constexpr int kZThreads = 1024;
constexpr int kZInFlight = 8;
__global__ __launch_bounds__(kZThreads) void zloss_kernel(const float* __restrict__ lse, int64_t T,
                                                          float* __restrict__ out) {
  __shared__ double part[kZThreads / 64];
  typedef __attribute__((ext_vector_type(4))) float f4;
  double acc = 0.0;
  const int64_t head_room = (int64_t)(((16u - ((uint32_t)(uintptr_t)lse & 15u)) & 15u) / 4u);
  const int64_t head = head_room < T ? head_room : T;
  const int64_t n4 = (T - head) / 4;
  if (threadIdx.x == 0) {
    for (int64_t i = 0; i < head; ++i) {
      const double v = lse[i];
      acc += v * v;
    }
  }
  const f4* const v4 = reinterpret_cast<const f4*>(lse + head);
  int64_t c = threadIdx.x;
  for (; c + (int64_t)(kZInFlight - 1) * kZThreads < n4; c += (int64_t)kZInFlight * kZThreads) {
    f4 q[kZInFlight];
#pragma unroll
    for (int u = 0; u < kZInFlight; ++u) q[u] = v4[c + (int64_t)u * kZThreads];
#pragma unroll
    for (int u = 0; u < kZInFlight; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc += (double)q[u][r] * (double)q[u][r];
  }
  for (; c < n4; c += kZThreads) {
    const f4 q = v4[c];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc += (double)q[r] * (double)q[r];
  }
  if (threadIdx.x == 0) {
    for (int64_t i = head + 4 * n4; i < T; ++i) {
      const double v = lse[i];
      acc += v * v;
    }
  }
  acc = wave_sum(acc);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kZThreads / 64; ++w) s += part[w];
    out[0] = T > 0 ? (float)(s / (double)T) : 0.0f;
  }
}

}  // namespace

hipError_t launch_balance_layers(const BalanceArgs& a, int n_layers, hipStream_t stream, hipEvent_t ev_stop) {
  return launch_timed(balance_layers_kernel, dim3((unsigned)n_layers), dim3(64), 0, stream, nullptr, ev_stop, a);
}

hipError_t launch_balance(const BalanceArgs& a, hipStream_t stream, hipEvent_t ev_stop) {
  return launch_balance_layers(a, 1, stream, ev_stop);
}

hipError_t launch_zloss(const float* lse, int64_t T, float* out, hipStream_t stream, hipEvent_t ev_stop) {
  return launch_timed(zloss_kernel, dim3(1), dim3(kZThreads), 0, stream, nullptr, ev_stop, lse, T, out);
}

}  // namespace elb
